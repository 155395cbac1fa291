"""Parity of a kernel's output with the oracle's, with the kernel's fp32
placement of the exponent as an explicit tolerance.

The oracle takes t = s - m~ exactly.  A kernel that forms the exponent in
fp32 (the fused kernel computes 2^23 (127 + R + t) as the fp32 output of the
score product, with its own fp32 frozen max) carries t to about 2^-16
binades.  Where the exact Mitchell value of an element lies within that of a
rounding tie, its code may fall on either side; where a block's largest
value lies that close to the tie that decides the block's binade, every
code of the block may be rounded one binade coarser or finer.  Each such
element may therefore move P~ by one grid step (two in a tied block), and
the row's output by those steps times |v^_j - out|, over l less the steps
(the flips may lower the row sum).

``excess_rel_l2`` removes exactly that allowance row by row and returns the
relative L2 of what is left, which is held to the same 2e-3 as everything
else.  Rows with no element near a tie get no allowance at all.
"""

import numpy as np

from oracle import FORMATS
from oracle.attention import mitchell_exp2, placement_exponent

# binades: the fp32 placement of t -- the accumulator start and the score
# product's two accumulation steps each round at 2^30..2^31, half an ulp
# being 2^-17 binades
EPS_PLACE = 3e-5

# The score product itself, per operand format, in binades per unit of the
# score's largest single product max_d |q'^_d k^_d|: with FP8 operands the
# matrix core's accumulation is not exact, and its error follows the largest
# product rather than the sum of all (measured on MI355X against exact
# scores, the kernel's frozen max of one-key rows: error / largest product at
# most 3.3e-4 over 131,072 products at D = 64 and 128, Gaussian keys and
# Student-t keys down to 1.5 degrees of freedom, scores up to 5,400 binades;
# error / absolute mass reached 2.6e-4 on the heaviest tails).  FP6 and FP4
# products came out exact (error 0 in every case).
SCORE_REL = {"e4m3": 5e-4}


def score_eps(info, fmt):
    """Per-element bound (binades) on the kernel's score error for operands
    in ``fmt``: 0, or SCORE_REL times a bound on the score's largest product,
    the lesser of max_d |q'^_d| * max_d |k^_d| and the absolute mass."""
    c = SCORE_REL.get(fmt, 0.0)
    if c == 0.0:
        return 0.0
    qa, ka = np.abs(info["q_hat"]), np.abs(info["k_hat"])
    return c * np.minimum(np.outer(qa.max(axis=1), ka.max(axis=1)), qa @ ka.T)


def eps_rows(gpu_m_tilde, info, fmt=None):
    """Margin of the kernel's t: its fp32 placement plus its frozen max's
    distance from the oracle's (held to fp32 rounding by the tests), per row;
    with the operand format ``fmt`` also each score's own product error, per
    element."""
    base = EPS_PLACE + np.abs(np.asarray(gpu_m_tilde, np.float64) - info["m_tilde"])
    se = 0.0 if fmt is None else score_eps(info, fmt)
    return base if np.isscalar(se) else base[:, None] + se


def frozen_max_tol(info, fmt=None):
    """Per-row bound on the kernel's frozen max against the oracle's.  It is
    mean + z std (or the window's max, or that max plus the 64-binade cap)
    evaluated in fp32 from the kernel's scores, so its rounding follows the
    magnitude of the window's scores, not of the guess itself (which can be
    near zero: two keys at -1.7 and -4.3).  With the operand format ``fmt``,
    each score also carries its product's own error (score_eps); the max, the
    mean and the spread each move by at most the window's largest, so the
    guess by at most 1 + z of it."""
    win = info["visible"][:, :128]
    mag = np.max(np.where(win, np.abs(info["scores"][:, :128]), 0.0), axis=1)
    tol = 1e-4 * np.maximum(1.0, np.maximum(np.abs(info["m_tilde"]), mag))
    se = 0.0 if fmt is None else score_eps(info, fmt)
    if not np.isscalar(se):
        n_vis = np.maximum(info["visible"].sum(axis=1), 1)
        z = np.sqrt(2.0 * np.log(n_vis)) + 1.0
        tol = tol + (1.0 + z) * np.max(np.where(win, se[:, :128], 0.0), axis=1)
    return tol


def kappa_eps(info, fmt, base=2e-3):
    """Per-row margin for a row's fallback offset: ``base``, plus the score
    error of its largest guess-relative score, plus the bound on the frozen
    max's own difference (frozen_max_tol), which moves every t of the row."""
    se = score_eps(info, fmt)
    mt = frozen_max_tol(info, fmt)
    if np.isscalar(se):
        return base + mt
    t = np.where(info["visible"], info["scores"] - info["m_tilde"][:, None], -np.inf)
    top = np.argmax(t, axis=1)
    return base + mt + se[np.arange(len(top)), top]


def tie_allowance(info, fmt, out_ref, eps_x, mode="block"):
    """Per-row bound on the output change that near-tie codes can cause;
    ``eps_x`` (binades: scalar, per row or per element) bounds how far the
    kernel's t may sit from the exact one; ``fmt`` and ``mode`` are P~'s
    format and variant."""
    f = FORMATS[fmt]
    M = f.mbits
    pl = placement_exponent(f)
    s, m, vis = info["scores"], info["m_tilde"], info["visible"]
    kap, delta = info["kappa"], info["delta"]
    R, S = s.shape
    t = s - m[:, None]
    dfull = np.repeat(delta, 32, axis=1)[:, :S]
    x = np.where(vis, t - kap[:, None] + pl + dfull, -np.inf)
    ea = np.asarray(eps_x, np.float64)
    if ea.ndim == 2:                                       # per element
        ex = ea
    else:                                                  # scalar or per row
        ex = np.broadcast_to(ea.reshape(-1, 1), (R, 1))
    if mode == "efq":
        # ties of the code-domain rounding: 2 x + 2 within 2 eps of k + 1/2
        with np.errstate(invalid="ignore"):
            c = 2.0 * x + 2.0
            lo = np.clip(np.floor(c), 0, f.max_code)
            near = vis & np.isfinite(c) & (np.abs(c - np.floor(c) - 0.5) <= 2.0 * ex) & (c > 0) & (c < f.max_code)
        from oracle import decode
        q = np.where(near, decode(np.minimum(lo + 1, f.max_code).astype(np.int64), f)
                     - decode(lo.astype(np.int64), f), 0.0)
    else:
        with np.errstate(over="ignore"):
            p = np.exp2(x) if mode == "exp" else mitchell_exp2(x)
        with np.errstate(divide="ignore", invalid="ignore"):
            e = np.floor(np.log2(np.where(p > 0, p, 1.0)))
            e = np.maximum(e, 1 - f.bias)                      # subnormal grid below emin
            q = np.ldexp(1.0, (e - M).astype(np.int64))
            r = p / q
            dist = np.abs(r - np.floor(r) - 0.5) * q           # value distance to the tie
            if mode == "exp":
                slope = p * np.log(2.0)
            else:
                slope = np.ldexp(1.0, np.floor(np.where(np.isfinite(x), x, 0.0)).astype(np.int64))
        near = vis & (p > 0) & (p < f.max_value) & (dist <= slope * ex)
    # blocks whose largest value decides its binade within eps_x of a tie
    nb = delta.shape[1]
    tp = np.full((R, nb * 32), -np.inf)
    tp[:, :S] = np.where(vis, t, -np.inf)
    tmax = tp.reshape(R, nb, 32).max(axis=2)
    if ex.shape[1] > 1:                                    # a block's margin: its largest
        ep = np.zeros((R, nb * 32))
        ep[:, :S] = ex
        ex = ep.reshape(R, nb, 32).max(axis=2)
    with np.errstate(invalid="ignore", over="ignore"):
        if mode == "exp":
            # the binade steps where 2^frac(t_max) rounds up to 2: 2^f = 2 - 2^-(M+1)
            f_up = np.log2(2.0 - 2.0 ** -(M + 1))
            fr = tmax - np.floor(np.where(np.isfinite(tmax), tmax, 0.0))
            tied = np.isfinite(tmax) & (np.abs(fr - f_up) <= ex)
        else:
            c = (2 ** M) * tmax
            k = np.rint((c + 0.5) / 2 ** M) * 2 ** M - 0.5
            tied = np.isfinite(c) & (np.abs(c - k) <= (2 ** M) * ex)
    tied_el = np.repeat(tied, 32, axis=1)[:, :S] & vis
    if mode == "row":
        tied_el[:] = False                                # no block shifts
    if mode == "efq":
        # a block one binade up or down moves x by -1 or +1 under twice or
        # half the scale: the element's value in this block's units becomes
        # 2 v(x - 1) or v(x + 1) / 2 (clamped codes included, which no code
        # tie covers)
        from oracle import decode

        def aff(xx):
            with np.errstate(invalid="ignore"):
                cc = np.rint(2.0 ** M * (xx + f.bias))
            return decode(np.clip(np.where(np.isfinite(cc), cc, 0.0), 0, f.max_code).astype(np.int64), f)
        v0 = aff(x)
        tstep = np.maximum(np.abs(2.0 * aff(x - 1.0) - v0), np.abs(0.5 * aff(x + 1.0) - v0))
    else:
        tstep = 2.0 * q
    step = np.where(near, q, 0.0) + np.where(tied_el, tstep, 0.0)
    step = step * np.ldexp(1.0, (-pl - dfull).astype(np.int64))
    # A set of flips delta_j (|delta_j| <= step_j) moves the row to
    # (O + sum delta_j v_j) / (l + sum delta_j), i.e. by
    # sum delta_j (v_j - out) / (l + sum delta_j): at most
    # sum step_j |v_j - out| / (l - sum step_j).
    vh = info["v_hat"]
    num = np.zeros(R)
    rows, cols = np.nonzero(step)
    for i, j in zip(rows, cols):
        num[i] += step[i, j] * np.linalg.norm(vh[j] - out_ref[i])
    l = info["l"]
    den = l - step.sum(axis=1)
    return np.where(num > 0, num / np.maximum(den, 1e-300), 0.0)


def excess_rel_l2(gpu_rows, ref_rows, info, fmt, eps_x, mode="block", skip=None):
    """Relative L2 of the part of the difference that near-tie codes cannot
    explain; also returns the number of rows that got an allowance.  Rows
    in ``skip`` (undecided(): the kernel took the other side of a fallback
    threshold that the row sits on) are not compared."""
    allow = tie_allowance(info, fmt, ref_rows, eps_x, mode)
    d = np.linalg.norm(np.asarray(gpu_rows) - np.asarray(ref_rows), axis=-1)
    ex = np.maximum(0.0, d - allow)
    if skip is not None:
        ex = np.where(np.asarray(skip), 0.0, ex)
    return float(np.linalg.norm(ex) / np.linalg.norm(ref_rows)), int(np.count_nonzero(allow))


def undecided(codes, gpu_kap, ref_kap):
    """Rows left free at a fallback threshold (kappa_rows code 2) on which the
    kernel and the oracle took different sides.  Whether such a row falls
    back at all hangs on a rounding tie within the kernel's own score error
    (with one scale per row: whether its top value rounds to the smallest
    subnormal code or to zero), and the two sides give different outputs,
    each right for its decision; such rows are compared on neither."""
    codes = np.asarray(codes).astype(np.int64)
    return ((codes & 2) != 0) & (np.asarray(gpu_kap) != np.asarray(ref_kap))
