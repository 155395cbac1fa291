"""Pins of the parity tolerance (tests/parity.py) on the CPU.

The GPU tests forgive exactly the output change that codes near a rounding
tie can make when t is placed to within eps binades.  These tests check that
bound against simulated kernels built from the oracle's own probability map:
a kernel whose t is off by a known amount is the oracle with its frozen max
moved by that amount (t = s - m~), so its codes flip exactly where the
exact value sits within that distance of a tie.

* an error within eps is absorbed in full (nothing is left over); eps is
  taken at 1e-3 binades here, where every format flips enough codes on a
  small head to exercise the bound (it is linear in eps; the kernel's own
  EPS_PLACE of 3e-5 flips too few FP6/FP4 codes on a CPU-sized sample);
* the same error with no allowance, or a much larger error, is not;
* a code moved one step away from any tie is not absorbed at all;
* FP8 score products: scores each off by up to their own bound (a fraction
  of their absolute mass) are absorbed by the per-element margin, and not
  by the per-row one alone.
"""

import numpy as np
import pytest

import workloads as W
import oracle as O
from oracle.attention import fused_probabilities
from parity import EPS_PLACE, SCORE_REL, excess_rel_l2, score_eps, tie_allowance

FMTS = ["e4m3", "e2m3", "e2m1"]


def _case(fmt, seed=91, S=512, rows=48, scale=1.6):
    q, k, v = (W.random_bf16((1, 1, S, 64), seed + i, scale) for i in range(3))
    qh, kh, vh = (W.bf16_bits_to_f64(x[0, 0]) for x in (q, k, v))
    _, info = O.fused_attention(qh, kh, vh, fmt, rows=np.arange(rows), return_info=True)
    out = info["P"] @ info["v_hat"] / info["l"][:, None]       # unrounded output rows
    return info, out


def _shifted(info, fmt, delta):
    """Output rows of a kernel whose t is larger by ``delta`` binades in
    every row (its frozen max lower by delta)."""
    fp = fused_probabilities(info["scores"], info["m_tilde"] - delta, info["visible"], fmt)
    P = fp["P"]
    return P @ info["v_hat"] / P.sum(axis=1)[:, None]


EPS = 1e-3


@pytest.mark.parametrize("fmt", FMTS)
def test_placement_error_within_eps_is_absorbed(fmt):
    info, out = _case(fmt)
    for delta in (0.8 * EPS, -0.8 * EPS):
        k_out = _shifted(info, fmt, delta)
        plain = O.rel_l2(k_out, out)
        ex, n_rows = excess_rel_l2(k_out, out, info, fmt, EPS)
        assert plain > 0.0 and n_rows > 0        # some codes did flip
        assert ex <= 1e-3 * plain, (delta, ex, plain)


@pytest.mark.parametrize("fmt", FMTS)
def test_without_allowance_nothing_is_forgiven(fmt):
    info, out = _case(fmt)
    k_out = _shifted(info, fmt, 0.8 * EPS)
    assert np.all(tie_allowance(info, fmt, out, 0.0) == 0.0)
    ex, n_rows = excess_rel_l2(k_out, out, info, fmt, 0.0)
    assert n_rows == 0
    assert ex == pytest.approx(O.rel_l2(k_out, out), rel=1e-12)


@pytest.mark.parametrize("fmt", FMTS)
def test_larger_placement_error_is_not_absorbed(fmt):
    info, out = _case(fmt)
    k_out = _shifted(info, fmt, 0.05)          # 50 x the allowed placement error
    plain = O.rel_l2(k_out, out)
    ex, _ = excess_rel_l2(k_out, out, info, fmt, EPS)
    assert ex >= 0.5 * plain > 0.0, (ex, plain)


@pytest.mark.parametrize("fmt", FMTS)
def test_code_moved_away_from_ties_is_not_absorbed(fmt):
    """The largest element of a row that has no element within the kernel's
    placement error of a tie is moved one grid step: the allowance gives
    that row nothing."""
    info, out = _case(fmt)
    f = O.FORMATS[fmt]
    allow = tie_allowance(info, fmt, out, EPS_PLACE)
    P = info["P"].copy()
    # a row with no allowance and an element of large weight
    i = int(np.flatnonzero(allow == 0.0)[0])
    j = int(np.argmax(P[i]))
    # one grid step at that element's binade, in P~ units
    step = np.ldexp(1.0, int(np.floor(np.log2(P[i, j]))) - f.mbits)
    P[i, j] -= step
    k_out = out.copy()
    k_out[i] = P[i] @ info["v_hat"] / P[i].sum()
    ex, _ = excess_rel_l2(k_out, out, info, fmt, EPS_PLACE)
    assert ex == pytest.approx(O.rel_l2(k_out, out), rel=1e-12)
    assert ex > 0.0


@pytest.mark.parametrize("fmt,mode", [(f, "block") for f in FMTS] + [("e2m1", "efq")])
def test_block_moved_across_its_binade_tie_is_absorbed(fmt, mode):
    """Each row's largest block has its largest value delta/2 above the tie
    that decides its binade, below the guess (so every row's offset stays
    0): a kernel with t lower by delta puts that whole block one binade lower
    and re-rounds every code on the other grid; the allowance covers it, and
    without its tied-block term it would not."""
    info0, _ = _case(fmt)
    M = O.FORMATS[fmt].mbits
    s, vis, vh = info0["scores"], info0["visible"], info0["v_hat"]
    R, S = s.shape
    delta = 0.8 * EPS
    t_tie = -1.0 - 2.0 ** -(M + 1)                 # binade -1 rounds up to 0 above this
    m = s.max(axis=1) - (t_tie + delta / 2)        # the row's largest score at the tie
    top = s.reshape(R, S // 32, 32).max(axis=2).argmax(axis=1)
    fp = fused_probabilities(s, m, vis, fmt, mode=mode)
    assert np.all(fp["kappa"] == 0)
    P = fp["P"]
    info = dict(fp)
    info.update(m_tilde=m, l=P.sum(axis=1), scores=s, v_hat=vh, visible=vis)
    out = P @ vh / info["l"][:, None]
    kp = fused_probabilities(s, m + delta, vis, fmt, mode=mode)
    rr = np.arange(R)
    assert np.all(kp["delta"][rr, top] == fp["delta"][rr, top] + 1)   # the top blocks moved
    k_out = kp["P"] @ vh / kp["P"].sum(axis=1)[:, None]
    plain = O.rel_l2(k_out, out)
    ex, _ = excess_rel_l2(k_out, out, info, fmt, EPS, mode)
    assert plain > 0.0 and ex <= 1e-3 * plain, (ex, plain)


def test_affine_block_moved_across_its_binade_tie_is_absorbed():
    """Affine E2M1 codes: one block whose largest score sits delta/2 below
    its binade tie, where its code is the clamped top one (no code tie to
    explain a change), its other scores away from any code tie.  A kernel
    with t higher by delta moves the whole block one binade up (its codes two
    steps down the affine line, under twice the scale); the allowance's
    tied-block term must cover it."""
    delta = 0.8 * EPS
    t = np.array([-1.25 - delta / 2, -1.6, -2.1, -3.3, -2.45, -1.9, -4.05, -2.8])
    s = np.concatenate([t, np.full(24, -9.3)])[None, :]
    vis = np.ones_like(s, bool)
    m = np.zeros(1)
    vh = np.random.default_rng(5).standard_normal((32, 16))
    fp = fused_probabilities(s, m, vis, "e2m1", mode="efq")
    kp = fused_probabilities(s, m - delta, vis, "e2m1", mode="efq")
    assert fp["kappa"][0] == 0 and kp["delta"][0, 0] == fp["delta"][0, 0] - 1
    assert fp["codes"][0, 0] == 7
    info = dict(fp)
    info.update(m_tilde=m, l=fp["P"].sum(axis=1), scores=s, v_hat=vh, visible=vis)
    out = fp["P"] @ vh / info["l"][:, None]
    k_out = kp["P"] @ vh / kp["P"].sum(axis=1)[:, None]
    plain = O.rel_l2(k_out, out)
    ex, _ = excess_rel_l2(k_out, out, info, "e2m1", EPS, "efq")
    assert plain > 1e-2 and ex <= 1e-3 * plain, (ex, plain)


def test_score_errors_within_their_bound_are_absorbed():
    """A simulated FP8 kernel whose every score is off by +-0.8 of its bound
    (SCORE_REL times the score's largest product, score_eps): the
    per-element margin absorbs the flips this causes; the per-row EPS_PLACE
    alone does not."""
    fmt = "e4m3"
    q, k, v = (W.random_bf16((1, 1, 512, 64), 95 + i, 3.0) for i in range(3))
    qh, kh, vh = (W.bf16_bits_to_f64(x[0, 0]) for x in (q, k, v))
    _, info = O.fused_attention(qh, kh, vh, fmt, rows=np.arange(48), return_info=True)
    out = info["P"] @ info["v_hat"] / info["l"][:, None]
    se = score_eps(info, fmt)
    assert SCORE_REL[fmt] > 0 and se.shape == info["scores"].shape
    sign = np.where(np.random.default_rng(5).random(se.shape) < 0.5, -1.0, 1.0)
    fp = fused_probabilities(info["scores"] + 0.8 * sign * se, info["m_tilde"], info["visible"], fmt)
    k_out = fp["P"] @ info["v_hat"] / fp["P"].sum(axis=1)[:, None]
    plain = O.rel_l2(k_out, out)
    assert plain > 0.0
    ex, _ = excess_rel_l2(k_out, out, info, fmt, EPS_PLACE + se)
    assert ex <= 1e-3 * plain, (ex, plain)
    ex0, _ = excess_rel_l2(k_out, out, info, fmt, EPS_PLACE)
    assert ex0 >= 0.1 * plain, (ex0, plain)


def test_undecided_rows_are_free_rows_with_different_offsets():
    """Only rows left free at a threshold (code 2, also with the borderline
    bit) whose offsets differ between the two sides escape the comparison."""
    from parity import undecided
    codes = np.array([0, 2, 2, 3, 1, 0])
    gpu = np.array([0, 0, 5, 1, 2, 4])
    ref = np.array([0, 0, 0, 0, 1, 0])
    assert undecided(codes, gpu, ref).tolist() == [False, False, True, True, False, False]


def test_offset_slack_follows_the_row_margin():
    """Borderline rows may differ by one, or by ceil(eps) where the margin
    spans binades; free rows not at all checked; others exactly."""
    from gpu_helpers import kappa_rows, check_kappa
    border = np.array([True, True, False, True])
    free = np.array([False, False, True, False])
    eps = np.array([0.3, 2.5, 0.0, 1e-3])
    codes = kappa_rows(border, free, eps)
    ref = np.array([100, 7000, 5, 0])
    check_kappa(ref + np.array([1, -3, 40, 1]), ref, codes)
    for bad in ([2, 0, 0, 0], [0, 4, 0, 0], [0, 0, 0, 2]):
        with pytest.raises(AssertionError):
            check_kappa(ref + np.array(bad), ref, codes)
    # a row that is neither borderline nor free must agree exactly
    plain = kappa_rows(np.zeros(4, bool), np.zeros(4, bool))
    with pytest.raises(AssertionError):
        check_kappa(ref + np.array([0, 0, 1, 0]), ref, plain)
