"""Attention references (oracle side; test infrastructure only).

Three results are computed, all on one (batch, head) slice with float64
arithmetic unless a step says otherwise:

* ``exact_attention`` -- softmax(q k^T / sqrt(D)) v on the unquantised bf16
  inputs: the ground truth the error criterion is measured against.
* ``plain_mx_attention`` -- the path that exponentiates, then quantises, on
  the very same MX operands as the fused path (the pre-scaled q' of step 1,
  k, v): exact row max, exact exponential, then the probabilities
  MX-quantised along the keys before the PV product.  Its error is what
  quantising the products' operands costs on its own, the bar the fused
  path's extra error is held under (Fused-Softmax for efficient quantized
  attention, summary; EFQ-Softmax: Exp-Free Quantization for Softmax,
  abstract), so that the
  fused/plain comparison isolates the approximated exponential and the
  frozen max.
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
   m~_i = fp32(min(max(w, mean + z_i * std), w + 64) + bias) with w the
   window max, population std, z_i = sqrt(2 ln n_i) + 1 with n_i the row's
   visible keys.  The pages fix no rule; the mean + z*std term is the
   expected Gaussian extreme over n_i keys plus one standard deviation of
   margin, so that a well-behaved row rarely exceeds it.  The cap of 64
   binades above the window max only binds on rows whose scores fall into
   far-apart clusters (a light upper tail): the row's top score is at least
   w, so the cap keeps every row within 65 binades below its guess, where
   the block shifts place it exactly.  ``bias`` (binades) is a test hook, 0
   in normal use.
4. The fast exponential is the bit-pattern one (``mitchell_exp2``): read as
   a float, the integer 2**23 * (127 + x) is 2**floor(x) * (1 + frac(x)),
   i.e. 2**x linearly interpolated between integer exponents.  Because x is
   linear in the score, the max subtraction and the scaling that produce it
   fold into the score product (its accumulator start and Q's block scale);
   that placement is the kernel's business, and here t_ij = s_ij - m~_i is
   taken exactly.
5. MX quantisation of P.  Per block b of 32 keys of a row (keys
   [32b, 32b+32), visible keys only), the block's binade relative to the
   guess, counted in element codes, is
   e_b = floor(round_half_even(2**M * max_j t_ij) / 2**M): the binade its
   largest value lands in once rounded to M mantissa bits.  The row's
   offset is kappa_i = max(0, max_b e_b) (step 6) and the block is shifted
   up by Delta_b = min(kappa_i - e_b, 127 - pl) whole binades (a fully
   masked block takes the largest shift), so that its largest value lands
   in the placement binade 2**pl: the top binade (pl = emax) for E2M3 and
   E2M1; for E4M3 the binade below it (pl = emax - 1), which keeps rounding
   away from E4M3's NaN pattern at no cost in precision (every normal E4M3
   binade has the same 3 mantissa bits).  Each element is
   mitchell_exp2(t_ij - kappa_i + pl + Delta_b) rounded to the nearest
   element (ties to even, saturating at the largest finite one), which puts
   values below the normal range on the subnormal grid by value.  The
   block's E8M0 scale is 2**-(pl + Delta_b) and
   P~_ij = decode(code_ij) * 2**-(pl + Delta_b), about 2**(t_ij - kappa_i).
6. Fallback: a row whose guess was too low has some block with e_b > 0
   (its scores exceed m~ by a whole binade in the code domain).  The row is
   recomputed with its reference raised by the whole number of binades
   kappa_i = max(0, max_b e_b).  Raising the reference by whole binades
   leaves every code of the row unchanged and lowers every block scale by
   2**kappa_i (except where a block shift reaches the E8M0 floor), so the
   recomputation is an exact power-of-two rescale of the row's sums.
7. O_i = sum_j P~_ij v^_j, l_i = sum_j P~_ij (the same quantised P~ in both,
   as EFQ-Softmax does for its numerator and denominator), and
   out_i = bf16(O_i / l_i).

Kernel tolerance.  A kernel that places x in fp32 (for instance as the
exponent-field value 2**23 * (127 + R + t) of a score product) carries t to
a fixed number of fraction bits; its codes and block binades then differ
from these exact ones only where the exact value lies within that rounding
of a rounding tie.  Parity tests absorb this in their tolerance.
"""

from __future__ import annotations

import math
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

from .mx import (FORMATS, BLOCK, Format, decode, encode_values, round_to_format,
                 mx_quantize, mx_dequantize, bf16_round)

WINDOW = 128          # keys that feed the frozen-max guess
Z_MARGIN = 1.0        # standard deviations above the expected Gaussian extreme
GUESS_CAP = 64.0      # largest lead of the guess over the window max, binades
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


def quantized_operands(q, k, v, fmt):
    """Dequantised q'^ (the pre-scaled q' of step 1), k^ (blocks along D) and
    v^ (blocks along keys): the operands both MX paths multiply."""
    f = _fmt(fmt)
    S = k.shape[0]
    qp = prescale_q(q)
    qh = mx_dequantize(*mx_quantize(qp, f), f)[:, : q.shape[1]]
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
    the "How it works" figure); the window, the extreme-value term, its
    margin and the cap over the window max are the reading taken here.
    """
    w = vis[:, :WINDOW]
    sw = s[:, :WINDOW]
    cnt = w.sum(axis=1)
    n_vis = vis.sum(axis=1)
    wmax = np.where(w, sw, -np.inf).max(axis=1)
    mean = np.where(w, sw, 0.0).sum(axis=1) / cnt
    var = np.where(w, (sw - mean[:, None]) ** 2, 0.0).sum(axis=1) / cnt
    z = np.sqrt(2.0 * np.log(n_vis)) + Z_MARGIN
    guess = np.minimum(np.maximum(wmax, mean + z * np.sqrt(var)), wmax + GUESS_CAP) + bias
    return guess.astype(np.float32).astype(np.float64)


def mitchell_exp2(x: np.ndarray) -> np.ndarray:
    """2**floor(x) * (1 + frac(x)): the bit-pattern exponential (step 4).

    Exact at integer x, at most about 6.1 % above 2**x in between.
    ``-inf`` gives 0.
    """
    x = np.asarray(x, np.float64)
    fin = np.isfinite(x)
    xs = np.where(fin, x, 0.0)
    fl = np.floor(xs)
    # floor(x) below the float64 exponent range underflows to 0, as it should
    val = np.ldexp(1.0 + (xs - fl), np.clip(fl, -1100, 1100).astype(np.int64))
    return np.where(fin, val, 0.0)


def placement_exponent(fmt) -> int:
    """Binade 2**pl in which a block's largest probability is placed: the top
    normal binade, except E4M3 where it is the one below (see step 5)."""
    f = _fmt(fmt)
    return f.emax - 1 if f.name == "e4m3" else f.emax


def block_binades(t: np.ndarray, vis: np.ndarray, fmt, exact: bool = False) -> np.ndarray:
    """e_b of step 5 for rows of guess-relative scores t [R, S]: the binade of
    each 32-key block's largest visible value after rounding to M mantissa
    bits (half to even).  Blocks with no visible key give -inf.  The value
    is the bit-pattern exponential's (its mantissa is frac(t), so the
    rounding is that of 2^M t), or with ``exact`` the exact 2^t's."""
    f = _fmt(fmt)
    R, S = t.shape
    nb = (S + BLOCK - 1) // BLOCK
    tp = np.full((R, nb * BLOCK), -np.inf)
    tp[:, :S] = np.where(vis, t, -np.inf)
    g = tp.reshape(R, nb, BLOCK).max(axis=2)
    with np.errstate(invalid="ignore", over="ignore"):
        if exact:
            fin = np.isfinite(g)
            e0 = np.floor(np.where(fin, g, 0.0))
            mant = np.exp2(np.where(fin, g, 0.0) - e0)          # 2^frac(t) in [1, 2)
            up = np.rint(mant * 2 ** f.mbits) >= 2 ** (f.mbits + 1)
            return np.where(fin, e0 + up, -np.inf)
        c = np.rint((2 ** f.mbits) * g)            # np.rint: half to even
    return np.floor(c / (2 ** f.mbits))


P_MODES = ("block", "row", "efq", "exp")


def overflow_threshold(fmt) -> float:
    """Smallest value that rounds beyond the format's largest finite element
    (the midpoint to the next grid point): 464 for E4M3."""
    f = _fmt(fmt)
    top = f.max_value
    return top + math.ldexp(1.0, int(math.floor(math.log2(top))) - f.mbits - 1)


def fused_probabilities(s: np.ndarray, m_tilde: np.ndarray, vis: np.ndarray,
                        fmt, mode: str = "block") -> Dict[str, np.ndarray]:
    """Steps 4-6 of the module doc for rows of log2-domain scores ``s`` [R, S].

    ``fmt`` is the element format of P~.  ``mode`` picks the P~ variant:

    * "block" (step 5): each 32-key block shifted to the placement binade.
    * "row": one scale for the whole row, Delta = 0 in every block (E4M3
      only: its 17 binades leave no block of a softmax row needing a shift
      of its own).  A row falls back when its largest value,
      mitchell_exp2(t_max + pl), reaches the format's overflow threshold
      (464 for E4M3: it would round beyond 448); it is then recomputed with
      kappa = max_b e_b whole binades.  Otherwise kappa = 0.
    * "efq" (E2M1 only): the codes come from a single affine rule in the
      code domain (EFQ-Softmax: Exp-Free Quantization for Softmax, abstract:
      an exponent-only block scale from the local maximum, then nonnegative
      E2M1 codes by one affine map of the shifted score).  With x as in
      step 5, code = clamp(round_half_even(2 x + 2), 0, 7): for values of
      1 and above this is the element the bit-pattern map rounds to; below,
      codes follow the line (x in [-0.75, -0.25) gives 0.5, lower gives 0).
    * "exp": as "block", with the exact exponential 2**x in place of the
      bit-pattern one, i.e. the rounding thresholds of the exact map (the
      threshold-corrected variant); a block's binade is then that of its
      largest exact value once rounded.

    Rows far below the guess fall back as well, re-based downwards by a
    negative kappa = max_b e_b: in the block modes a row whose top block
    needs a shift beyond 127 - pl binades (its scale would clamp, leaving
    the block off the placement binade and, further down, the row sum at 0
    or below fp32's range); with one scale per row a row whose codes would
    all be zero (l = 0, the output 0/0).

    Returns the P~ values (float64), the element codes, the per-block shifts
    Delta, the E8M0 scale bytes of P~, the per-row binade offset kappa
    (> 0 for rows that fell back) and the guess-relative block binades e_b.
    """
    f = _fmt(fmt)
    if mode not in P_MODES:
        raise ValueError("unknown P~ mode " + repr(mode))
    if mode == "row" and f.name != "e4m3":
        raise ValueError("the one-scale-per-row P~ is defined for E4M3")
    if mode == "efq" and f.name != "e2m1":
        raise ValueError("the affine-rule P~ is defined for E2M1")
    pl = placement_exponent(f)
    cap = 127 - pl
    R, S = s.shape
    t = np.asarray(s, np.float64) - np.asarray(m_tilde, np.float64)[:, None]
    e = block_binades(t, vis, f, exact=(mode == "exp"))
    emax = np.max(e, axis=1) if e.size else np.full(R, -np.inf)
    if mode == "row":
        tmax = np.where(vis, t, -np.inf).max(axis=1) if S else np.full(R, -np.inf)
        with np.errstate(over="ignore"):
            over = mitchell_exp2(tmax + pl) >= overflow_threshold(f)
        kappa = np.where(over, emax, 0.0)
    else:
        # a top block beyond the largest shift (more than cap binades below
        # the guess) is re-based downwards so that it lands in the placement
        # binade all the same
        low = np.isfinite(emax) & (emax < -cap)
        kappa = np.where(low, emax, np.maximum(0.0, emax))

    def place(kappa):
        if mode == "row":
            delta = np.zeros_like(e)
        else:
            delta = np.where(np.isfinite(e), np.minimum(kappa[:, None] - e, cap), cap)
        delta_full = np.repeat(delta, BLOCK, axis=1)[:, :S]
        x = np.where(vis, t - kappa[:, None] + pl + delta_full, -np.inf)
        if mode == "efq":
            with np.errstate(invalid="ignore"):
                c = np.rint(2.0 ** f.mbits * (x + f.bias))
            code = np.clip(np.where(np.isfinite(c), c, 0.0), 0, f.max_code).astype(np.int64)
            vals = decode(code, f)
        else:
            with np.errstate(over="ignore"):
                p = np.exp2(x) if mode == "exp" else mitchell_exp2(x)
            vals = round_to_format(p, f)
            code = encode_values(vals, f).astype(np.int64)
        return delta, code, vals * np.ldexp(1.0, (-pl - delta_full).astype(np.int32))

    delta, code, P = place(kappa)
    # one scale per row: rows whose every code flushed, re-based downwards
    # by their top binade (the block modes never get here: their top block
    # always lands in the placement binade)
    flush = (P.sum(axis=1) == 0.0) & vis.any(axis=1) & np.isfinite(emax)
    if flush.any():
        kappa = np.where(flush, emax, kappa)
        delta, code, P = place(kappa)
    return {
        "P": P,
        "codes": code,
        "delta": delta.astype(np.int64),
        "scale_bytes": (127 - pl - delta).astype(np.int64),
        "kappa": kappa.astype(np.int64),
        "binades": e,
    }


def fused_attention(q, k, v, fmt, causal: bool = False, rows=None, bias: float = 0.0,
                    return_info: bool = False, p_fmt=None, p_mode: str = "block"):
    """Fused-Softmax attention output (bf16 values as float64) for one head.

    ``q, k, v`` are [S, D] arrays of bf16 values; ``rows`` selects query rows
    (all by default); ``bias`` is added to the frozen max (binades).  ``fmt``
    is the element format of q'^, k^ and v^; ``p_fmt`` that of P~ (the same
    by default; E4M3 P~ over FP6/FP4 operands is the mixed variant) and
    ``p_mode`` its variant (see ``fused_probabilities``).  With
    ``return_info`` also returns the frozen max, the fallback offsets, the
    log2-domain scores, the P~ values, the dequantised q'^, k^ and v^ and the
    visibility.
    """
    f = _fmt(fmt)
    pf = f if p_fmt is None else _fmt(p_fmt)
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    S, D = k.shape
    rows = _rows(rows, S)
    qh, kh, vh = quantized_operands(q[rows] if rows.size else q[:0], k, v, f)
    s = qh @ kh.T
    vis = _visible(rows, S, causal)
    m_tilde = frozen_max(s, vis, bias)
    fp = fused_probabilities(s, m_tilde, vis, pf, p_mode)
    P = fp["P"]
    O = P @ vh
    l = P.sum(axis=1)
    out = bf16_round(O / l[:, None])
    if not return_info:
        return out
    info = dict(fp)
    info.update(m_tilde=m_tilde, l=l, scores=s, q_hat=qh, k_hat=kh, v_hat=vh, visible=vis)
    return out, info


def plain_probabilities(s: np.ndarray, vis: np.ndarray, fmt) -> np.ndarray:
    """Exp-then-quantize probabilities for rows of log2-domain scores [R, S]:
    P = 2**(s - max_j s) with the exact row max, then MX-quantised along the
    keys (blocks of 32 aligned at key 0, the OCP rule of ``mx_quantize``) in
    the operand format.  Masked keys are 0.  Returns the dequantised values."""
    f = _fmt(fmt)
    S = s.shape[1]
    sm = np.where(vis, s, -np.inf)
    m = sm.max(axis=1, keepdims=True)
    P = np.where(vis, np.exp2(sm - m), 0.0)
    return mx_dequantize(*mx_quantize(P, f), f)[:, :S]


def plain_mx_attention(q, k, v, fmt, causal: bool = False, rows=None,
                       return_info: bool = False, p_fmt=None):
    """Exp-then-quantize attention (bf16 values as float64) for one head.

    The same MX operands as ``fused_attention`` (q'^ of step 1, k^, v^), so
    the same log2-domain scores s; exact row max and exact exponential in
    float64, P = 2**(s - max s) = exp((q'.k - max) ...) in the softmax scale;
    P MX-quantised along the keys (``plain_probabilities``);
    out = bf16(sum P^ v^ / sum P^).  ``p_fmt`` is the format of P^ (that of
    the operands by default).  With ``return_info`` also returns the
    dequantised P^ and the scores.
    """
    f = _fmt(fmt)
    pf = f if p_fmt is None else _fmt(p_fmt)
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    S, D = k.shape
    rows = _rows(rows, S)
    qh, kh, vh = quantized_operands(q[rows], k, v, f)
    s = qh @ kh.T
    vis = _visible(rows, S, causal)
    Pq = plain_probabilities(s, vis, pf)
    O = Pq @ vh
    l = Pq.sum(axis=1)
    out = bf16_round(O / l[:, None])
    if not return_info:
        return out
    return out, {"P": Pq, "scores": s}
