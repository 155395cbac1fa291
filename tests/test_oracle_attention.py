"""Pins for the oracle's attention references (CPU only).

The checks come from outside the oracle's own formulas: a second, loop-based
exact attention; closed forms (V = 1 gives 1, Q = 0 gives the mean of V);
a hand-worked frozen-max example; the bit-pattern exponential evaluated by a
different route (math.ldexp and a brute-force nearest search); exactness at
integer exponents; causal rows equal to shorter non-causal problems; planted
outliers that must fall back; and the error criterion of the method
(fused error within 1.1x the exp-then-quantize error) on the small workload.
"""

import math
import os

import numpy as np
import pytest

import workloads as W
import oracle as O
from oracle import FORMATS, decode, mx_quantize, mx_dequantize, bf16_round, rel_l2
from oracle.attention import (frozen_max, fused_probabilities, score_scale, prescale_q,
                              quantized_operands, _visible, WINDOW, mitchell_exp2,
                              placement_exponent)

FMTS = ["e4m3", "e2m3", "e2m1"]
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _head(S, D, seed, scale=1.0):
    return [W.bf16_bits_to_f64(W.random_bf16((S, D), seed + i, scale)) for i in range(3)]


def test_exact_attention_matches_loops():
    q, k, v = _head(7, 3, 100)
    D = 3
    for causal in (False, True):
        ref = np.zeros((7, 3))
        for i in range(7):
            js = range(i + 1) if causal else range(7)
            sc = [sum(q[i, d] * k[j, d] for d in range(D)) / math.sqrt(D) for j in js]
            m = max(sc)
            w = [math.exp(x - m) for x in sc]
            tot = sum(w)
            for d in range(D):
                ref[i, d] = sum(wj * v[j, d] for wj, j in zip(w, js)) / tot
        got = O.exact_attention(q, k, v, causal)
        assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)
    # first causal row sees only key 0
    assert np.array_equal(O.exact_attention(q, k, v, True)[0], v[0])


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("causal", [False, True])
def test_fused_v_ones_gives_ones(fmt, causal):
    q, k, _ = _head(96, 64, 200, scale=1.5)
    v = np.ones_like(q)
    out = O.fused_attention(q, k, v, fmt, causal)
    assert np.array_equal(out, np.ones_like(out))
    out = O.plain_mx_attention(q, k, v, fmt, causal)
    assert np.array_equal(out, np.ones_like(out))


@pytest.mark.parametrize("fmt", FMTS)
def test_fused_q_zero_gives_mean_of_quantised_v(fmt):
    _, k, v = _head(80, 64, 300)
    q = np.zeros_like(k)
    vh = mx_dequantize(*mx_quantize(np.ascontiguousarray(v.T), fmt), fmt)[:, :80].T
    want = bf16_round(vh.sum(axis=0) / 80.0)
    out, info = O.fused_attention(q, k, v, fmt, return_info=True)
    assert np.array_equal(out, np.broadcast_to(want, out.shape))
    assert np.all(info["P"] == 1.0)
    assert np.all(info["kappa"] == 0)


def test_frozen_max_worked_example():
    lines = dict(l.split(None, 1) for l in open(os.path.join(GOLDEN, "frozen_max_example.txt"))
                 if l.strip() and not l.startswith("#"))
    S = int(lines["S"])
    expected = float(lines["expected"])
    s = np.zeros((1, S))
    s[0, :WINDOW] = np.where(np.arange(WINDOW) % 2 == 0, 1.0, -1.0)
    s[0, WINDOW:] = 3.0            # beyond the window: must not matter
    vis = np.ones((1, S), bool)
    got = frozen_max(s, vis)[0]
    assert got == float(np.float32(got))
    assert abs(got - expected) < 1e-6
    # a window max above the extreme-value term wins
    s[0, 5] = 9.0
    assert frozen_max(s, vis)[0] == 9.0


def test_frozen_max_capped_example():
    """Two far-apart clusters in the window: the extreme-value term would
    put the guess 440 binades above the window max; the cap holds it at 64
    above (hand-worked golden), and a bias adds after the cap."""
    lines = dict(l.split(None, 1) for l in open(os.path.join(GOLDEN, "frozen_max_capped_example.txt"))
                 if l.strip() and not l.startswith("#"))
    S = int(lines["S"])
    expected = float(lines["expected"])
    s = np.zeros((1, S))
    s[0, :WINDOW] = np.where(np.arange(WINDOW) % 2 == 0, 100.0, -100.0)
    s[0, WINDOW:] = -500.0
    vis = np.ones((1, S), bool)
    assert frozen_max(s, vis)[0] == expected
    assert frozen_max(s, vis, bias=-8.0)[0] == expected - 8.0
    # every row of a block map then stays within its largest shift: no row
    # falls back, and the top block lands in the placement binade
    for fmt in FMTS:
        fp = fused_probabilities(s, frozen_max(s, vis), vis, fmt)
        assert fp["kappa"][0] == 0 and fp["delta"][0].min() == 64


def _mitchell_value(x):
    """2**floor(x) * (1 + frac(x)) via math, not via bit patterns."""
    fl = math.floor(x)
    return math.ldexp(1.0 + (x - fl), fl)


def _nearest(vals_table, a):
    dist = np.abs(vals_table - a)
    cand = np.flatnonzero(dist == dist.min())
    return vals_table[cand[0]] if cand.size == 1 else vals_table[[c for c in cand if c % 2 == 0][0]]


@pytest.mark.parametrize("mode", ["block", "exp"])
@pytest.mark.parametrize("fmt", FMTS + ["e3m2"])
def test_probability_map_against_independent_route(fmt, mode):
    """P~ of single-block rows, recomputed with math.ldexp (bit-pattern
    exponential) or math.pow (the exact one) and brute-force rounding from
    the exact score differences."""
    f = FORMATS[fmt]
    rng = np.random.default_rng(17)
    R = 64
    s = rng.normal(0, 4, size=(R, 32))                 # log2-domain scores
    m = (s.max(axis=1) + rng.uniform(0.0, 6.0, R)).astype(np.float32).astype(np.float64)
    vis = np.ones((R, 32), bool)
    fp = fused_probabilities(s, m, vis, f, mode=mode)
    expo = _mitchell_value if mode == "block" else (lambda x: math.pow(2.0, x))
    table = decode(np.arange(f.max_code + 1), f)
    pl = f.emax - 1 if fmt == "e4m3" else f.emax
    M = f.mbits
    for i in range(R):
        t = s[i] - m[i]
        if mode == "block":
            # block binade from the largest score, in element codes (half to even)
            x = (2 ** M) * max(t)
            code = round(x)                             # Python rounds half to even
            e = math.floor(code / 2 ** M)
        else:
            # binade of the largest exact value once its mantissa is rounded
            mant, ex = math.frexp(2.0 ** max(t))        # 2^t = mant * 2^ex, mant in [0.5, 1)
            e = ex - 1 + (round(2 * mant * 2 ** M) == 2 ** (M + 1))
        delta = min(-e, 127 - pl)
        assert fp["kappa"][i] == 0
        assert fp["delta"][i, 0] == delta
        for j in range(32):
            p = expo(pl + delta + t[j])
            want = _nearest(table, min(p, f.max_value * 2)) * 2.0 ** (-pl - delta)
            assert fp["P"][i, j] == want, (i, j)


@pytest.mark.parametrize("fmt", FMTS)
def test_probability_exact_at_integer_exponents_and_bounded(fmt):
    f = FORMATS[fmt]
    # scores whose log2-probability relative to the guess is an integer
    ks = np.array([0, -1, -2, -3, -1, 0, -2, -1] * 4, dtype=np.float64)
    s = ks[None, :]
    m = np.zeros(1)
    fp = fused_probabilities(s, m, np.ones_like(s, bool), f)
    # with no subnormal flush (E2M1 keeps 3 binades), P~ == 2**k exactly
    keep = ks >= -(f.emax + f.bias - 1)
    assert np.array_equal(fp["P"][0][keep], np.exp2(ks[keep]))
    # monotone in the score, and within the Mitchell + rounding band for normal codes
    s = np.sort(np.random.default_rng(1).normal(0, 1, (1, 32)))
    mx = np.array([s.max()]).astype(np.float32).astype(np.float64)
    fp = fused_probabilities(s, mx, np.ones_like(s, bool), f)
    P = fp["P"][0]
    assert np.all(np.diff(P) >= 0)
    t = s[0] - mx[0]
    pl = f.emax - 1 if fmt == "e4m3" else f.emax
    # elements whose value before rounding is in the normal range
    unrounded = np.array([_mitchell_value(pl + fp["delta"][0, 0] + x) for x in t])
    normal = unrounded >= 2.0 ** (1 - f.bias)
    ratio = P[normal] / np.exp2(t[normal])
    half_ulp = 2.0 ** -(f.mbits + 1)
    assert np.all(ratio >= 1.0 / (1.0 + half_ulp) - 1e-6)
    assert np.all(ratio <= 1.0615 * (1.0 + half_ulp) + 1e-6)


@pytest.mark.parametrize("fmt", FMTS)
def test_v_power_of_two_and_column_order(fmt):
    """V enters only through its MX blocks along the keys: scaled by 2^k it
    keeps its codes (the output scales exactly), and its columns permuted
    permute the output's columns.  A V quantised along D instead, or a scale
    applied to the wrong column, fails one of the two."""
    q, k, v = _head(96, 64, 600)
    base = O.fused_attention(q, k, v, fmt, causal=True)
    for e in (-90, 33):
        assert np.array_equal(O.fused_attention(q, k, v * 2.0 ** e, fmt, causal=True), base * 2.0 ** e)
    perm = np.random.default_rng(601).permutation(64)
    assert np.array_equal(O.fused_attention(q, k, v[:, perm], fmt, causal=True), base[:, perm])


def test_causal_row_equals_shorter_noncausal_problem():
    q, k, v = _head(192, 64, 400)
    for fmt in FMTS:
        full = O.fused_attention(q, k, v, fmt, causal=True)
        for i in (31, 63, 127, 191):       # i+1 a multiple of 32: identical V blocks
            n = i + 1
            short = O.fused_attention(q[:n], k[:n], v[:n], fmt, causal=False, rows=[i])
            assert np.array_equal(full[i], short[0]), (fmt, i)


def test_planted_outliers_fall_back():
    w = W.WORKLOADS["outliers_e2m1"]
    q, k, v = [W.bf16_bits_to_f64(a) for a in W.generate_head(w, 0, 0, S=4096)]
    # regenerate the outlier rows for this shorter problem
    import dataclasses
    ws = dataclasses.replace(w, S=4096)
    rows = W.outlier_rows(ws, 0, 0)
    assert rows.size == 40
    out, info = O.fused_attention(q, k, v, "e2m1", rows=rows, return_info=True)
    # the planted score is +8 sigma of the row (q keeps its norm): it always
    # exceeds the guess by more than the top binade's headroom
    assert np.mean(info["kappa"] > 0) >= 0.97
    # after the fallback the rows are as accurate as exp-then-quantize ones
    ex = O.exact_attention(q, k, v, rows=rows)
    pl = O.plain_mx_attention(q, k, v, "e2m1", rows=rows)
    assert rel_l2(out, ex) <= 1.25 * rel_l2(pl, ex)


@pytest.mark.parametrize("fmt", FMTS)
def test_forced_fallback_matches_normal_rows(fmt):
    """A guess far too low makes every row fall back; results stay equivalent."""
    q, k, v = _head(256, 64, 500)
    base, i0 = O.fused_attention(q, k, v, fmt, return_info=True)
    low, i1 = O.fused_attention(q, k, v, fmt, bias=-8.0, return_info=True)
    assert np.all(i0["kappa"] == 0) and np.all(i1["kappa"] > 0)
    ex = O.exact_attention(q, k, v)
    # the two differ only in the rounding phase of the codes: equally accurate
    assert 0.8 * rel_l2(base, ex) <= rel_l2(low, ex) <= 1.2 * rel_l2(base, ex)


def test_error_criterion_on_tiny_workload():
    w = W.WORKLOADS["tiny"]
    qs, ks, vs = W.generate(w)
    fused, plain, exact = [], [], []
    for h in range(w.H):
        q, k, v = (W.bf16_bits_to_f64(a[0, h]) for a in (qs, ks, vs))
        fused.append(O.fused_attention(q, k, v, "e4m3"))
        plain.append(O.plain_mx_attention(q, k, v, "e4m3"))
        exact.append(O.exact_attention(q, k, v))
    fused, plain, exact = map(np.concatenate, (fused, plain, exact))
    e_f, e_p = rel_l2(fused, exact), rel_l2(plain, exact)
    assert e_p < 0.1
    assert e_f <= 1.1 * e_p


def test_score_scale_and_prescale():
    """The fp32 constants of step 1 against independent evaluations."""
    from fractions import Fraction
    for D in (64, 128):
        c = score_scale(D)
        assert c == float(np.float32(c))
        assert abs(c * math.sqrt(D) * math.log(2.0) - 1.0) < 1e-7
        q = W.bf16_bits_to_f64(W.random_bf16((4, D), 5, 3.0))
        qp = prescale_q(q)
        for a, b in zip(q.ravel()[:64], qp.ravel()[:64]):
            # one fp32 rounding of the exact product
            assert b == float(np.float32(Fraction(a) * Fraction(c)))


def test_mitchell_exp2_closed_forms():
    """2**floor(x) * (1 + frac x): exact at integers, the chord of 2**x in between."""
    xs = np.array([0.0, 1.0, -3.0, 0.5, -0.25, 2.75, -7.125, -np.inf])
    want = [1.0, 2.0, 0.125, 1.5, 0.875, 7.0, 2.0 ** -8 * 1.875, 0.0]
    assert np.array_equal(mitchell_exp2(xs), np.array(want))
    x = np.random.default_rng(3).uniform(-30, 30, 10000)
    r = mitchell_exp2(x) / np.exp2(x)
    assert np.all(r >= 1.0 - 1e-15) and np.all(r <= 1.0615)


def _loop_plain_rows(s, vis, fmt):
    """Exp-then-quantize probabilities by explicit loops: exact exponential of
    each score against its row's visible maximum, then each block of 32
    consecutive keys of a row MX-quantised on its own (OCP floor scale,
    brute-force nearest value, ties to the even code)."""
    f = FORMATS[fmt]
    mags = decode(np.arange(f.max_code + 1), f)
    R, S = s.shape
    out = np.zeros((R, S))
    for i in range(R):
        m = max(s[i, j] for j in range(S) if vis[i, j])
        p = [math.pow(2.0, s[i, j] - m) if vis[i, j] else 0.0 for j in range(S)]
        for b0 in range(0, S, 32):
            blk = p[b0:b0 + 32]
            amax = max(blk)
            if amax == 0.0:
                continue
            X = math.frexp(amax)[1] - 1 - f.emax
            for jj, val in enumerate(blk):
                y = val / 2.0 ** X
                d = np.abs(mags - min(y, f.max_value))
                cand = np.flatnonzero(d == d.min())
                c = cand[0] if cand.size == 1 else [c for c in cand if c % 2 == 0][0]
                out[i, b0 + jj] = mags[c] * 2.0 ** X
    return out


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("causal", [False, True])
def test_plain_probabilities_match_loops(fmt, causal):
    """The exp-then-quantize floor: P^ blocked along the keys of each row, in the
    operand format, from 2**(s - row max); and its output O / l."""
    S, D = 75, 64                       # a ragged third key block
    q, k, v = _head(S, D, 600, scale=1.4)
    rows = np.array([0, 1, 2, 17, 40, 74])
    out, info = O.plain_mx_attention(q, k, v, fmt, causal, rows=rows, return_info=True)
    vis = _visible(rows, S, causal)
    want = _loop_plain_rows(info["scores"], vis, fmt)
    assert np.array_equal(info["P"], want)
    # the scores are those of the fused path (the same pre-scaled q'^)
    _, finfo = O.fused_attention(q, k, v, fmt, causal, rows=rows, return_info=True)
    assert np.array_equal(info["scores"], finfo["scores"])
    _, _, vh = quantized_operands(q, k, v, fmt)
    for r in range(rows.size):
        num = [math.fsum(want[r, j] * vh[j, d] for j in range(S)) for d in range(D)]
        den = math.fsum(want[r])
        ref = bf16_round(np.array(num) / den)
        # one bf16 rounding apart at most (summation order)
        assert np.all(np.abs(out[r] - ref) <= np.abs(ref) * 2.0 ** -7 + 1e-30)


@pytest.mark.parametrize("fmt", FMTS)
def test_whole_binade_guess_shift_is_exact(fmt):
    """Lowering the guess by K whole binades (the fallback's re-basing) raises
    kappa by exactly K and leaves every code and every P~ unchanged."""
    f = FORMATS[fmt]
    rng = np.random.default_rng(21)
    R, S = 8, 96
    s = rng.normal(0.0, 1.5, (R, S))
    # guesses a hair above each row max: top block in binade 0, kappa = 0
    m = s.max(axis=1) + 2.0 ** -(f.mbits + 3)
    vis = np.ones((R, S), bool)
    base = fused_probabilities(s, m, vis, f)
    assert np.all(base["kappa"] == 0)
    for K in (1, 3, 17, 60):
        sh = fused_probabilities(s, m - K, vis, f)
        assert np.all(sh["kappa"] == K)
        assert np.array_equal(sh["codes"], base["codes"])
        assert np.array_equal(sh["P"], base["P"])
        assert np.array_equal(sh["delta"], base["delta"])



# ---- P~ variants (see fused_probabilities) ----

def test_variant_row_scale_closed_form_and_fallback():
    """One scale per row: every element is mitchell(t + pl) rounded, with no
    block shift; a row falls back exactly when its largest value reaches
    464 (it would round past 448) or rounds to zero (every code flushed),
    and then by its top block's binade."""
    f = FORMATS["e4m3"]
    table = decode(np.arange(f.max_code + 1), f)
    rng = np.random.default_rng(31)
    s = rng.normal(0.0, 3.0, (8, 64))
    m = s.max(axis=1) + np.array([0.3, 0.0, -0.5, -1.8, -1.9, -4.0, 18.0, 25.0])
    vis = np.ones_like(s, bool)
    fp = fused_probabilities(s, m, vis, "e4m3", mode="row")
    assert np.all(fp["delta"] == 0)
    for i in range(8):
        t = s[i] - m[i]
        over = _mitchell_value(max(t) + 7) >= 464.0
        flush = _nearest(table, _mitchell_value(max(t) + 7)) == 0.0
        assert fp["kappa"][i] == (math.floor(round(8 * max(t)) / 8) if over or flush else 0), i
        for j in range(64):
            want = _nearest(table, min(_mitchell_value(t[j] - fp["kappa"][i] + 7), 896.0)) * 2.0 ** -7
            assert fp["P"][i, j] == want, (i, j)
    assert list(fp["kappa"][:3]) == [0, 0, 0] and fp["kappa"][4] >= 1 and fp["kappa"][5] >= 4
    # 18 and 25 binades above the row: every code would flush; the fallback
    # brings the top block back to the placement binade
    assert fp["kappa"][6] <= -18 and fp["kappa"][7] <= -25
    assert np.all(fp["P"][6:].max(axis=1) >= 1.0)


def test_variant_row_scale_fallback_forgets_the_guess():
    """A row that falls back, on either side (guess 48 binades low: its top
    value overflows; 32 or 40 binades high: every code flushes), is
    recomputed from its own top binade, so its output no longer depends on
    the guess.  The biases keep every guess in one fp32 binade, [32, 64) in
    magnitude, so that the guesses differ by whole binades exactly."""
    q, k, v = (W.random_bf16((200, 64), 300 + j, 1.0) for j in range(3))
    qh, kh, vh = (W.bf16_bits_to_f64(x) for x in (q, k, v))
    res = {b: O.fused_attention(qh, kh, vh, "e4m3", bias=b, return_info=True, p_mode="row")
           for b in (-48.0, 32.0, 40.0)}
    out0, info0 = O.fused_attention(qh, kh, vh, "e4m3", bias=0.0, return_info=True, p_mode="row")
    assert np.all((info0["m_tilde"] >= 0.0) & (info0["m_tilde"] < 16.0))
    for b, (o, info) in res.items():
        assert np.all(np.isfinite(o)) and np.all(info["l"] > 0)
        assert np.array_equal(o, res[32.0][0]), b
        assert np.array_equal(info["kappa"], res[32.0][1]["kappa"] + 32 - int(b)), b
    assert np.all(res[32.0][1]["kappa"] < 0) and np.all(res[-48.0][1]["kappa"] > 0)


@pytest.mark.parametrize("fmt,mode", [("e4m3", "block"), ("e2m3", "block"), ("e2m1", "block"),
                                      ("e4m3", "exp"), ("e2m1", "efq")])
def test_flushed_rows_fall_back_like_rows_far_above(fmt, mode):
    """A guess 144 or 176 binades above every row puts each block beyond the
    largest shift (127 - pl binades): every code would flush and l = 0.
    Such rows are re-based downwards by their top binade (kappa < 0), which
    makes them the same rows as with the guess 144 binades below (kappa > 0,
    re-based upwards): identical outputs, offsets apart by the whole
    binades between the guesses.  The biases keep every guess in one fp32
    binade, [128, 256) in magnitude, so that they differ by whole binades
    exactly."""
    q, k, v = (W.random_bf16((160, 64), 340 + j, 1.0) for j in range(3))
    qh, kh, vh = (W.bf16_bits_to_f64(x) for x in (q, k, v))
    okw = dict(p_mode=mode) if mode != "block" else {}
    _, info0 = O.fused_attention(qh, kh, vh, fmt, bias=0.0, return_info=True, **okw)
    assert np.all(np.abs(info0["m_tilde"]) < 16.0)
    res = {b: O.fused_attention(qh, kh, vh, fmt, bias=b, return_info=True, **okw)
           for b in (-144.0, 144.0, 176.0)}
    for b, (o, info) in res.items():
        assert np.all(np.isfinite(o)) and np.all(info["l"] > 0), b
        assert np.array_equal(o, res[-144.0][0]), b
        assert np.array_equal(info["kappa"], res[-144.0][1]["kappa"] - 144 - int(b)), b
    assert np.all(res[-144.0][1]["kappa"] > 0) and np.all(res[144.0][1]["kappa"] < 0)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m3", "e2m1"])
def test_top_block_always_lands_in_the_placement_binade(fmt):
    """The invariant the fallback keeps in the block map: in every row, its
    largest value, in units of its block's scale, lies in the placement
    binade [2^pl, 2^(pl+1)), whether the row sits above its guess, near it,
    or far below it (guesses from 200 binades below the row to 500 above it,
    across the largest shift of 127 - pl binades and past the 189 binades
    that the scores' fp32 bit patterns reach)."""
    f = FORMATS[fmt]
    pl = O.attention.placement_exponent(f)
    rng = np.random.default_rng(41)
    s = rng.normal(0.0, 2.0, (400, 96))
    top = s.max(axis=1)
    # guess-relative top scores spread over [-500, 200], with rows packed
    # around the low threshold -(127 - pl)
    off = np.concatenate([rng.uniform(-500, 200, 200), -(127 - pl) + rng.uniform(-2, 2, 200)])
    m = top - off
    vis = np.ones_like(s, bool)
    fp = fused_probabilities(s, m, vis, fmt)
    dfull = np.repeat(fp["delta"], 32, axis=1)[:, :96]
    vals = fp["P"] * np.ldexp(1.0, (pl + dfull).astype(np.int64))
    vmax = vals.max(axis=1)
    assert np.all((vmax >= 2.0 ** pl) & (vmax < 2.0 ** (pl + 1))), (off[vmax < 2.0 ** pl][:5])
    # below the threshold the rows re-base downwards, above it they do not
    assert np.all(fp["kappa"][off < -(127 - pl) - 1] < 0)
    assert np.all(fp["kappa"][(off > -(127 - pl) + 1) & (off < 0)] == 0)


def test_variant_affine_codes_closed_form():
    """Affine E2M1 codes: the default map wherever the value is 1 or more
    (in units of the block's placement), the straight line below it."""
    rng = np.random.default_rng(32)
    s = rng.normal(0.0, 2.0, (16, 96))
    m = (s.max(axis=1) + rng.uniform(0, 3, 16)).astype(np.float32).astype(np.float64)
    vis = np.ones_like(s, bool)
    aff = fused_probabilities(s, m, vis, "e2m1", mode="efq")
    ref = fused_probabilities(s, m, vis, "e2m1")
    assert np.array_equal(aff["delta"], ref["delta"]) and np.array_equal(aff["kappa"], ref["kappa"])
    x = s - m[:, None] + 2 + np.repeat(ref["delta"], 32, axis=1)[:, :96]
    hi = x >= 0.0
    assert np.array_equal(aff["codes"][hi], ref["codes"][hi])
    # below 1: code 1 (0.5) on [-0.75, -0.25), code 2 (1.0) from -0.25, 0 under -0.75
    lo = ~hi
    want = np.where(x >= -0.25, 2, np.where(x >= -0.75, 1, 0))
    exact_tie = np.isclose((2 * x + 2) % 1.0, 0.5)
    assert np.array_equal(aff["codes"][lo & ~exact_tie], want[lo & ~exact_tie])
    # monotone in the score within a block
    for i in range(16):
        o = np.argsort(s[i, :32])
        assert np.all(np.diff(aff["P"][i, :32][o]) >= 0)


@pytest.mark.parametrize("variant", [("e4m3", dict(p_mode="row")), ("e2m3", dict(p_fmt="e4m3")),
                                     ("e2m1", dict(p_fmt="e4m3")), ("e2m1", dict(p_mode="efq")),
                                     ("e4m3", dict(p_mode="exp")), ("e2m1", dict(p_mode="exp")),
                                     ("e2m3", dict(p_fmt="e3m2"))])
def test_variants_v_ones_and_q_zero(variant):
    fmt, kw = variant
    q, k, v = _head(96, 64, 700, scale=1.5)
    out = O.fused_attention(q, k, np.ones_like(v), fmt, **kw)
    assert np.array_equal(out, np.ones_like(out))
    vh = mx_dequantize(*mx_quantize(np.ascontiguousarray(v.T), fmt), fmt)[:, :96].T
    out = O.fused_attention(np.zeros_like(q), k, v, fmt, **kw)
    assert np.array_equal(out, np.broadcast_to(bf16_round(vh.sum(axis=0) / 96.0), out.shape))


def test_e4m3_probabilities_over_fp4_operands_are_more_accurate():
    """E4M3 P~ over FP4 operands: the same operands as the FP4 default, a
    finer P~; its error against exact attention is lower."""
    w = W.WORKLOADS["tiny"]
    q, k, v = (W.bf16_bits_to_f64(a[0, 0]) for a in W.generate(w))
    ex = O.exact_attention(q, k, v)
    e_mix = rel_l2(O.fused_attention(q, k, v, "e2m1", p_fmt="e4m3"), ex)
    e_fp4 = rel_l2(O.fused_attention(q, k, v, "e2m1"), ex)
    assert e_mix < e_fp4


def test_e3m2_probabilities_keep_more_binades_with_coarser_steps():
    """E3M2 P~ (placement 2^4, smallest step 2^-4) against E2M3 (placement
    2^2, smallest step 2^-3), on one block whose top score sits at the
    guess: both give 1 there; 2^-6 survives only in E3M2 (E2M3 flushes
    anything below 2^-6 of the block's top); near the top E3M2's two
    mantissa bits are coarser (the bit-pattern value 0.95 of t = -0.1
    rounds to 0.9375 in E2M3 and to 1 in E3M2); 2^-9 is half of E3M2's
    smallest step and rounds to zero (ties to even), 1.5 * 2^-9 up to it."""
    t = np.array([0.0, -0.1, -6.0, -9.0, -8.5, -2.0])
    s = np.full((1, 32), -60.0)
    s[0, : t.size] = t
    m = np.zeros(1)
    vis = np.ones_like(s, bool)
    p6 = fused_probabilities(s, m, vis, "e2m3")["P"][0, : t.size]
    p5 = fused_probabilities(s, m, vis, "e3m2")["P"][0, : t.size]
    assert list(p6) == [1.0, 0.9375, 0.0, 0.0, 0.0, 0.25]
    assert list(p5) == [1.0, 1.0, 2.0 ** -6, 0.0, 2.0 ** -8, 0.25]


def test_error_criterion_on_clustered_keys():
    """Keys in two opposite clusters put the extreme-value guess far above
    every row, where the cap holds it 64 binades over the window max: the
    rows are placed by block shifts alone, and the fused error stays within
    1.1x the plain quantised path's on every head and format."""
    q, k, v = W.two_valued_keys(1, 2, 512, 128, seed=3)
    rows = np.arange(0, 512, 8)
    for fmt in FMTS:
        for h in range(2):
            qh, kh, vh = (W.bf16_bits_to_f64(x[0, h]) for x in (q, k, v))
            exa = O.exact_attention(qh, kh, vh, rows=rows)
            fu, info = O.fused_attention(qh, kh, vh, fmt, rows=rows, return_info=True)
            pl = O.plain_mx_attention(qh, kh, vh, fmt, rows=rows)
            assert np.all(info["kappa"] == 0)
            assert rel_l2(fu, exa) <= 1.1 * rel_l2(pl, exa), (fmt, h)
