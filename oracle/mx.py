"""MX element formats and block quantisation (oracle side; test infrastructure only).

The pages name the operand formats only as MXFP8, MXFP6 and MXFP4
(Fused-Softmax for efficient quantized attention, summary) and E2M1
(EFQ-Softmax: Exp-Free Quantization for Softmax, abstract).  The encodings
below are those of the OCP Microscaling Formats (MX) v1.0 specification:

* FP8 E4M3: 1 sign, 4 exponent bits (bias 7), 3 mantissa bits, no infinity,
  the all-ones pattern is NaN, largest finite 448.
* FP6 E2M3: 1 sign, 2 exponent bits (bias 1), 3 mantissa bits, largest 7.5.
* FP6 E3M2: 1 sign, 3 exponent bits (bias 3), 2 mantissa bits, largest 28
  (the other FP6 element type of the OCP specification; here only a
  probability format, not an operand format of the attention path).
* FP4 E2M1: 1 sign, 2 exponent bits (bias 1), 1 mantissa bit, largest 6.
* E8M0 scale: an unsigned byte X+127 meaning 2**X; 0xFF is NaN.

A block is 32 consecutive elements sharing one scale.  The block scale is
the OCP rule: X = floor(log2(amax)) - emax, where emax is the exponent of
the format's largest normal; X is clamped to [-127, 127]; an all-zero block
takes X = -127.  Elements are x / 2**X rounded to the nearest representable
value, ties to an even mantissa, and values beyond the largest finite
magnitude saturate to it (never NaN).  Readings taken where the OCP text
leaves a choice: saturation (not NaN) on overflow, the input's sign bit is
kept on zero results, a block holding NaN or Inf gets scale byte 0xFF and
all-zero codes, and a partial tail block takes its amax over its valid
elements with zero codes in the padding.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Dict, Tuple

import numpy as np

BLOCK = 32


@dataclasses.dataclass(frozen=True)
class Format:
    name: str
    ebits: int
    mbits: int
    bias: int
    max_code: int      # largest finite magnitude code (sign bit clear)

    @property
    def bits(self) -> int:
        return 1 + self.ebits + self.mbits

    @property
    def emin(self) -> int:
        """Exponent of the smallest normal binade."""
        return 1 - self.bias

    @property
    def max_value(self) -> float:
        return float(_magnitude_table(self)[self.max_code])

    @property
    def emax(self) -> int:
        """Exponent of the largest normal binade (floor(log2(max_value)))."""
        return int(math.floor(math.log2(self.max_value)))


FORMATS: Dict[str, Format] = {
    "e4m3": Format("e4m3", 4, 3, 7, 0x7E),
    "e2m3": Format("e2m3", 2, 3, 1, 0x1F),
    "e2m1": Format("e2m1", 2, 1, 1, 0x07),
    "e3m2": Format("e3m2", 3, 2, 3, 0x1F),
}


def _fmt(f) -> Format:
    return f if isinstance(f, Format) else FORMATS[f]


def _magnitude_table(f: Format) -> np.ndarray:
    """Value of every magnitude code 0 .. 2**(ebits+mbits)-1 (sign bit clear)."""
    n = 1 << (f.ebits + f.mbits)
    vals = np.empty(n, np.float64)
    for c in range(n):
        e = c >> f.mbits
        m = c & ((1 << f.mbits) - 1)
        if e == 0:
            vals[c] = math.ldexp(m, f.emin - f.mbits)               # subnormal
        else:
            vals[c] = math.ldexp((1 << f.mbits) + m, e - f.bias - f.mbits)
    if f.name == "e4m3":
        vals[n - 1] = np.nan                                         # S.1111.111
    return vals


def decode(codes: np.ndarray, fmt) -> np.ndarray:
    """Float64 value of element codes (sign bit = bit ``bits-1``)."""
    f = _fmt(fmt)
    codes = np.asarray(codes).astype(np.int64)
    mag = codes & ((1 << (f.ebits + f.mbits)) - 1)
    sign = (codes >> (f.ebits + f.mbits)) & 1
    v = _magnitude_table(f)[mag]
    return np.where(sign == 1, -v, v)


def _floor_log2(a: np.ndarray) -> np.ndarray:
    """floor(log2(a)) for finite a > 0, exactly (via the binary exponent)."""
    _, e = np.frexp(a)
    return e.astype(np.int64) - 1


def round_to_format(y: np.ndarray, fmt) -> np.ndarray:
    """Round float64 values onto the format's grid: nearest, ties to even
    mantissa, saturating at the largest finite magnitude.  Input must be finite.
    """
    f = _fmt(fmt)
    y = np.asarray(y, np.float64)
    a = np.abs(y)
    safe = np.where(a > 0, a, 1.0)
    e = np.maximum(np.where(a > 0, _floor_log2(safe), f.emin), f.emin)
    quantum = np.ldexp(1.0, (e - f.mbits).astype(np.int32))
    r = np.rint(a / quantum) * quantum          # np.rint rounds half to even
    r = np.minimum(r, f.max_value)
    return np.copysign(r, y)


def encode_values(vals: np.ndarray, fmt) -> np.ndarray:
    """Codes of values that lie exactly on the grid (sign from the sign bit)."""
    f = _fmt(fmt)
    table = _magnitude_table(f)[: f.max_code + 1]
    a = np.abs(vals)
    mag = np.searchsorted(table, a)
    if not np.all(table[np.minimum(mag, f.max_code)] == a):
        raise ValueError("value not representable in " + f.name)
    sign = np.signbit(vals).astype(np.int64)
    return (mag | (sign << (f.ebits + f.mbits))).astype(np.uint8)


def mx_quantize(x: np.ndarray, fmt) -> Tuple[np.ndarray, np.ndarray]:
    """MX-quantise along the last axis in blocks of 32 (OCP MX v1.0 rule).

    ``x`` holds float64 values (normally exact bf16 values), shape
    ``[..., n]``.  Returns ``(codes, scales)``: one code per byte, shape
    ``[..., ceil(n/32)*32]`` with zero codes in the padding, and E8M0 scale
    bytes, shape ``[..., ceil(n/32)]``.
    """
    f = _fmt(fmt)
    x = np.asarray(x, np.float64)
    n = x.shape[-1]
    nb = (n + BLOCK - 1) // BLOCK
    pad = nb * BLOCK - n
    xp = np.concatenate([x, np.zeros(x.shape[:-1] + (pad,))], axis=-1) if pad else x
    xb = xp.reshape(x.shape[:-1] + (nb, BLOCK))
    finite = np.isfinite(xb)
    bad = ~finite.all(axis=-1)
    xb = np.where(finite, xb, 0.0)
    amax = np.abs(xb).max(axis=-1)
    X = np.where(amax > 0, _floor_log2(np.where(amax > 0, amax, 1.0)) - f.emax, -127)
    X = np.clip(X, -127, 127)
    y = np.ldexp(xb, (-X)[..., None].astype(np.int32))      # exact power-of-two scaling
    codes = encode_values(round_to_format(y, f), f)
    scales = (X + 127).astype(np.uint8)
    codes[bad] = 0
    scales[bad] = 0xFF
    return codes.reshape(x.shape[:-1] + (nb * BLOCK,)), scales


def mx_dequantize(codes: np.ndarray, scales: np.ndarray, fmt) -> np.ndarray:
    """Float64 values of MX codes (one code per byte) and E8M0 scales."""
    vals = decode(codes, fmt)
    nb = scales.shape[-1]
    vb = vals.reshape(vals.shape[:-1] + (nb, BLOCK))
    s = scales.astype(np.int64)
    mult = np.where(s == 0xFF, np.nan, np.ldexp(1.0, (s - 127).astype(np.int32)))
    return (vb * mult[..., None]).reshape(vals.shape)


def pack_codes(codes: np.ndarray, fmt) -> np.ndarray:
    """Bytes of codes in memory order.

    FP8: one byte per element.  FP6: a little-endian bit stream, element i at
    bits [6i, 6i+6) of its 32-element block (24 bytes per block).  FP4: two
    elements per byte, the lower-indexed element in the low nibble.
    """
    f = _fmt(fmt)
    c = np.asarray(codes).astype(np.uint32)
    if f.bits == 8:
        return c.astype(np.uint8)
    if f.bits == 4:
        c2 = c.reshape(c.shape[:-1] + (-1, 2))
        return (c2[..., 0] | (c2[..., 1] << 4)).astype(np.uint8)
    # FP6: every 4 elements make 24 bits = 3 bytes.
    c4 = c.reshape(c.shape[:-1] + (-1, 4))
    w = c4[..., 0] | (c4[..., 1] << 6) | (c4[..., 2] << 12) | (c4[..., 3] << 18)
    out = np.stack([w & 0xFF, (w >> 8) & 0xFF, (w >> 16) & 0xFF], axis=-1)
    return out.reshape(c.shape[:-1] + (-1,)).astype(np.uint8)


def unpack_codes(packed: np.ndarray, fmt, n: int) -> np.ndarray:
    """Inverse of ``pack_codes`` for ``n`` elements along the last axis."""
    f = _fmt(fmt)
    p = np.asarray(packed).astype(np.uint32)
    if f.bits == 8:
        return p[..., :n].astype(np.uint8)
    if f.bits == 4:
        lo, hi = p & 0xF, p >> 4
        return np.stack([lo, hi], axis=-1).reshape(p.shape[:-1] + (-1,))[..., :n].astype(np.uint8)
    p3 = p.reshape(p.shape[:-1] + (-1, 3))
    w = p3[..., 0] | (p3[..., 1] << 8) | (p3[..., 2] << 16)
    c = np.stack([(w >> (6 * i)) & 0x3F for i in range(4)], axis=-1)
    return c.reshape(p.shape[:-1] + (-1,))[..., :n].astype(np.uint8)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bfloat16 (nearest, ties to even), as float64.

    bfloat16 has 8 significant bits and float32's exponent range; below
    2**-126 the quantum is 2**-133.  Overflow goes to infinity.
    """
    x = np.asarray(x, np.float64)
    a = np.abs(x)
    safe = np.where((a > 0) & np.isfinite(a), a, 1.0)
    e = np.maximum(_floor_log2(safe), -126)
    quantum = np.ldexp(1.0, (e - 7).astype(np.int32))
    r = np.rint(a / quantum) * quantum
    r = np.where(r >= 2.0 ** 128, np.inf, r)
    r = np.where(np.isfinite(a) & (a > 0), r, a)
    return np.copysign(r, x)
