"""Attention references (oracle side; test infrastructure only).

Three results are computed, all on one (batch, head) slice with float64
arithmetic unless a step says otherwise:

* ``exact_attention`` -- softmax(q k^T / sqrt(D)) v on the unquantised bf16
  inputs: the ground truth the error criterion is measured against.
* ``plain_mx_attention`` -- the "exp-then-quantize" path: MX operands, exact
  max and exact exp, then the probabilities MX-quantised before the PV
  product.  Its error is the floor set by quantising the GEMM operands
  (Fused-Softmax for efficient quantized attention, summary; EFQ-Softmax:
  Exp-Free Quantization for Softmax, abstract).
* ``fused_attention`` -- Fused-Softmax attention as specified below.

Fused-Softmax, as the pages outline it and as read here
-------------------------------------------------------
The pages say that softmax is reformulated and approximated so that its
dominant work folds into the attention GEMMs: the max subtraction and the
exponential go into the score product, the exponential is approximated "with
a fast method" and fused with the MX quantisation of P, probabilities are
summed on the matrix cores, and the row max is frozen speculatively with a
fallback when the guess is wrong (Fused-Softmax for efficient quantized
attention, summary; Moving softmax to matrix operations speeds up AI
inference by over 2x, "Read it as" and the "How it works" figure).  They give
no formulas, so each step below is a reading:

1. The softmax scale goes into Q: q' = fp32(q * c) with
   c = fp32(log2(e) / sqrt(D)), so that scores come out in binades of the
   probability.  q' and k are MX-quantised along D, v along the key axis
   (blocks of 32 keys aligned at key 0): the MX blocks lie along each
   product's reduction axis.
2. s_ij = sum_d q'^_id k^_jd (log2-domain scores).  Key j is visible to row i
   if j < S and, when causal, j <= i.
3. Frozen max (``frozen_max``): from the visible keys among the first 128,
   m~_i = fp32(max(window max, mean + z_i * std) + bias), population std,
   z_i = sqrt(2 ln n_i) + 1 with n_i the row's visible keys.  The pages fix
   no rule; the mean + z*std term is the expected Gaussian extreme over n_i
   keys plus one standard deviation of margin, so that a well-behaved row
   rarely exceeds it.  ``bias`` (binades) is a test hook, 0 in normal use.
4. Exponential folded into the score product.  The float32 number whose bit
   pattern is the integer 2**23 * (127 + x) has the value
   2**floor(x) * (1 + frac(x)), i.e. 2**x linearly interpolated between
   integer exponents (the bit-pattern exponential).  The score product itself
   produces that integer: with 2**23 folded into q's power-of-two block scale
   and the accumulator started at fp32(2**23 * (127 + R - kappa_i - m~_i)),
       y_ij = fp32(2**23 * s_ij + fp32(2**23 * (127 + R - kappa_i) - 2**23 * m~_i)),
   one rounding at the product's output (R = 62, below).  Truncation to an
   unsigned integer (0 below zero) gives the bits of
   p_ij = 2**(t_ij + R - kappa_i), t_ij = s_ij - m~_i, with 16 or more
   fraction bits of t.  R only places the value inside fp32's range: scores
   from 188 binades below the reference to 66 above give normal numbers.
5. MX quantisation of P.  Per block b of 32 keys of a row (keys
   [32b, 32b+32), visible keys only), with y0 the kappa = 0 values of step 4,
   c_b = round_half_even(2**M * (max_j y0_ij / 2**23 - 127 - R)) and
   e_b = floor(c_b / 2**M): the binade of the block's largest value relative
   to the guess, counted in element codes.  The block is shifted up by
   Delta_b = min(kappa_i - e_b, 127 - pl) whole binades so that its largest
   value lands in the placement binade 2**pl: the top binade (pl = emax) for
   E2M3 and E2M1; for E4M3 the binade below it (pl = emax - 1), which keeps
   rounding away from E4M3's NaN pattern at no cost in precision (every
   normal E4M3 binade has the same 3 mantissa bits).  Each element is
   p_ij * 2**(pl + Delta_b - R) (an exact power-of-two rescale) rounded to
   the nearest element (ties to even, saturating at the largest finite one),
   which puts values below the normal range on the subnormal grid by value.
   The block's E8M0 scale is 2**-(pl + Delta_b) and
   P~_ij = decode(code_ij) * 2**-(pl + Delta_b), about 2**(t_ij - kappa_i).
6. Fallback: a row whose guess was too low has some block with e_b > 0
   (its scores exceed m~ by a whole binade in the code domain).  The row is
   recomputed with its reference raised by the whole number of binades
   kappa_i = max(0, max_b e_b).  Raising the reference by whole binades
   leaves every code of the row unchanged (up to the fp32 rounding of y) and
   lowers every block scale by 2**kappa_i (except where a block shift
   reaches the E8M0 floor), so the kernel can realise the recomputation as
   an exact power-of-two rescale of its running sums.
7. O_i = sum_j P~_ij v^_j, l_i = sum_j P~_ij (the same quantised P~ in both,
   as EFQ-Softmax does for its numerator and denominator), and
   out_i = bf16(O_i / l_i).
"""

from __future__ import annotations

import math
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

from .mx import (FORMATS, BLOCK, Format, decode, encode_values, round_to_format,
                 mx_quantize, mx_dequantize, bf16_round)

WINDOW = 128          # keys that feed the frozen-max guess
Z_MARGIN = 1.0        # standard deviations above the expected Gaussian extreme
REF_BINADE = 62       # R of step 4: where a score equal to the reference lands
LOG2E = 1.0 / math.log(2.0)


def rel_l2(a: np.ndarray, b: np.ndarray) -> float:
    """||a - b||_2 / ||b||_2 over all elements."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm((a - b).ravel()) / np.linalg.norm(b.ravel()))


def _fmt(f) -> Format:
    return f if isinstance(f, Format) else FORMATS[f]


def _rows(rows, S) -> np.ndarray:
    return np.arange(S) if rows is None else np.asarray(rows, np.int64)


def _visible(rows: np.ndarray, S: int, causal: bool) -> np.ndarray:
    j = np.arange(S)[None, :]
    if causal:
        return j <= rows[:, None]
    return np.ones((rows.size, S), dtype=bool)


def score_scale(D: int) -> float:
    """c = fp32(log2(e) / sqrt(D)): the softmax scale in binades (step 1)."""
    return float(np.float32(LOG2E / math.sqrt(D)))


def prescale_q(q: np.ndarray) -> np.ndarray:
    """q' = fp32(q * c), element by element in fp32 (step 1)."""
    c = np.float32(score_scale(q.shape[1]))
    return (np.asarray(q, np.float64).astype(np.float32) * c).astype(np.float64)


def quantized_operands(q, k, v, fmt, prescale: bool = False):
    """Dequantised q^ (of q' when ``prescale``), k^ (blocks along D) and
    v^ (blocks along keys)."""
    f = _fmt(fmt)
    S = k.shape[0]
    if prescale:
        q = prescale_q(q)
    qh = mx_dequantize(*mx_quantize(q, f), f)[:, : q.shape[1]]
    kh = mx_dequantize(*mx_quantize(k, f), f)[:, : k.shape[1]]
    vt = mx_dequantize(*mx_quantize(np.ascontiguousarray(v.T), f), f)[:, :S]
    return qh, kh, np.ascontiguousarray(vt.T)


def exact_attention(q, k, v, causal: bool = False, rows=None) -> np.ndarray:
    """float64 softmax(q k^T / sqrt(D)) v for one head; q, k, v are [S, D]."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    S, D = k.shape
    rows = _rows(rows, S)
    s = (q[rows] @ k.T) / math.sqrt(D)
    vis = _visible(rows, S, causal)
    s = np.where(vis, s, -np.inf)
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=1, keepdims=True)
    return p @ v


def frozen_max(s: np.ndarray, vis: np.ndarray, bias: float = 0.0) -> np.ndarray:
    """Speculative row max from the first WINDOW keys (step 3 of the module doc).

    ``s``: float64 scores [R, S]; ``vis``: visibility [R, S].  Returns fp32
    values as float64.  The pages say only that the max is fixed
    speculatively and frozen before the fused product (Moving softmax to
    matrix operations speeds up AI inference by over 2x, "Read it as" and
    the "How it works" figure); the window, the extreme-value term and its
    margin are this build's reading.
    """
    w = vis[:, :WINDOW]
    sw = s[:, :WINDOW]
    cnt = w.sum(axis=1)
    n_vis = vis.sum(axis=1)
    wmax = np.where(w, sw, -np.inf).max(axis=1)
    mean = np.where(w, sw, 0.0).sum(axis=1) / cnt
    var = np.where(w, (sw - mean[:, None]) ** 2, 0.0).sum(axis=1) / cnt
    z = np.sqrt(2.0 * np.log(n_vis)) + Z_MARGIN
    guess = np.maximum(wmax, mean + z * np.sqrt(var)) + bias
    return guess.astype(np.float32).astype(np.float64)


def fma_f32(a: np.ndarray, b: np.ndarray, c: np.ndarray) -> np.ndarray:
    """fp32 fused multiply-add of fp32 operands, rounded once (nearest, ties even).

    a*b is exact in float64; a + c is resolved with an error-free two-sum so
    that the single rounding to fp32 is exact even on float64 ties.
    """
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    c = np.asarray(c, np.float64)
    p = a * b
    s = p + c
    bb = s - p
    err = (p - (s - bb)) + (c - bb)
    with np.errstate(invalid="ignore", over="ignore"):
        r = s.astype(np.float32).astype(np.float64)
        up = r > s
        other = np.where(up, np.nextafter(r.astype(np.float32), np.float32(-np.inf)),
                         np.nextafter(r.astype(np.float32), np.float32(np.inf))).astype(np.float64)
        lo = np.where(up, other, r)
        hi = np.where(up, r, other)
        tie = np.isfinite(s) & ((s - lo) == (hi - s))
    r = np.where(tie & (err > 0), hi, np.where(tie & (err < 0), lo, r))
    return r


def bits_to_f32(u: np.ndarray) -> np.ndarray:
    """float32 value (as float64) of unsigned 32-bit patterns."""
    return np.asarray(u, np.uint64).astype(np.uint32).view(np.float32).astype(np.float64)


def trunc_u32(y: np.ndarray) -> np.ndarray:
    """Truncate toward zero to an unsigned 32-bit integer; below zero or NaN give 0."""
    y = np.asarray(y, np.float64)
    y = np.where(np.isnan(y), 0.0, y)
    return np.clip(np.trunc(y), 0, 2.0 ** 32 - 1).astype(np.uint64)


def placement_exponent(fmt) -> int:
    """Binade 2**pl in which a block's largest probability is placed: the top
    normal binade, except E4M3 where it is the one below (see step 5)."""
    f = _fmt(fmt)
    return f.emax - 1 if f.name == "e4m3" else f.emax


def reference_addend(m_tilde: np.ndarray, kappa: np.ndarray) -> np.ndarray:
    """fp32(2**23 * (127 + R - kappa) - 2**23 * m~): the accumulator start of
    the score product (step 4), one rounding."""
    a = (2.0 ** 23) * (127 + REF_BINADE - np.asarray(kappa, np.float64)) - (2.0 ** 23) * m_tilde
    return a.astype(np.float32).astype(np.float64)


def exponent_field_values(s: np.ndarray, addend: np.ndarray) -> np.ndarray:
    """y = fp32(2**23 * s + addend) for rows of log2-domain scores (step 4)."""
    return fma_f32(np.float64(2.0 ** 23), s, addend[:, None])


def fused_probabilities(s: np.ndarray, m_tilde: np.ndarray, vis: np.ndarray,
                        fmt) -> Dict[str, np.ndarray]:
    """Steps 4-6 of the module doc for rows of log2-domain scores ``s`` [R, S].

    Returns the P~ values (float64), the element codes, the per-block shifts
    Delta, the E8M0 scale bytes of P~ and the per-row binade offset kappa
    (> 0 for rows that fell back).
    """
    f = _fmt(fmt)
    M = f.mbits
    pl = placement_exponent(f)
    cap = 127 - pl
    R, S = s.shape
    nb = (S + BLOCK - 1) // BLOCK
    s0 = np.where(vis, s, 0.0)
    # guess-relative block binades from the kappa = 0 values
    y0 = exponent_field_values(s0, reference_addend(m_tilde, np.zeros(R)))
    yp = np.full((R, nb * BLOCK), -np.inf)
    yp[:, :S] = np.where(vis, y0, -np.inf)
    g = yp.reshape(R, nb, BLOCK).max(axis=2)          # -inf for blocks with no visible key
    c = np.rint((2 ** M) * (g / 2.0 ** 23 - 127 - REF_BINADE))   # exact in float64
    e = np.floor(c / (2 ** M))
    kappa = np.maximum(0.0, np.max(e, axis=1))
    delta = np.where(np.isfinite(e), np.minimum(kappa[:, None] - e, cap), cap)
    delta_full = np.repeat(delta, BLOCK, axis=1)[:, :S]
    y = exponent_field_values(s0, reference_addend(m_tilde, kappa))
    y = np.where(vis, y, -np.inf)
    p = bits_to_f32(trunc_u32(y))
    p = p * np.ldexp(1.0, (pl + delta_full - REF_BINADE).astype(np.int32))
    vals = round_to_format(p, f)
    code = encode_values(vals, f).astype(np.int64)
    P = vals * np.ldexp(1.0, (-pl - delta_full).astype(np.int32))
    return {
        "P": P,
        "codes": code,
        "delta": delta.astype(np.int64),
        "scale_bytes": (127 - pl - delta).astype(np.int64),
        "kappa": kappa.astype(np.int64),
    }


def fused_attention(q, k, v, fmt, causal: bool = False, rows=None, bias: float = 0.0,
                    return_info: bool = False):
    """Fused-Softmax attention output (bf16 values as float64) for one head.

    ``q, k, v`` are [S, D] arrays of bf16 values; ``rows`` selects query rows
    (all by default); ``bias`` is added to the frozen max (binades).  With
    ``return_info`` also returns the frozen max, the fallback offsets, the
    log2-domain scores and the P~ values.
    """
    f = _fmt(fmt)
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    S, D = k.shape
    rows = _rows(rows, S)
    qh, kh, vh = quantized_operands(q[rows] if rows.size else q[:0], k, v, f, prescale=True)
    s = qh @ kh.T
    vis = _visible(rows, S, causal)
    m_tilde = frozen_max(s, vis, bias)
    fp = fused_probabilities(s, m_tilde, vis, f)
    P = fp["P"]
    O = P @ vh
    l = P.sum(axis=1)
    out = bf16_round(O / l[:, None])
    if not return_info:
        return out
    info = dict(fp)
    info.update(m_tilde=m_tilde, l=l, scores=s)
    return out, info


def plain_mx_attention(q, k, v, fmt, causal: bool = False, rows=None) -> np.ndarray:
    """Exp-then-quantize attention (bf16 values as float64) for one head.

    The same MX operands as ``fused_attention``; exact row max and exact exp
    in float64; P MX-quantised along the keys (blocks of 32 aligned at key 0,
    the same blocks as the fused path); out = bf16(sum P^ v^ / sum P^).
    """
    f = _fmt(fmt)
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    S, D = k.shape
    rows = _rows(rows, S)
    qh, kh, vh = quantized_operands(q[rows], k, v, f)
    s = qh @ kh.T
    vis = _visible(rows, S, causal)
    s = np.where(vis, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    P = np.where(vis, np.exp((s - m) / math.sqrt(D)), 0.0)
    Pq = mx_dequantize(*mx_quantize(P, f), f)[:, :S]
    O = Pq @ vh
    l = Pq.sum(axis=1)
    return bf16_round(O / l[:, None])
