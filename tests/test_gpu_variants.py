"""P~ variants (fsa_options.p_variant) on the GPU against the oracle's
definitions (oracle.attention.fused_probabilities modes):

* "row"       one scale per row, E4M3;
* "e4m3"      E4M3 P~ over FP6/FP4 operands (mixed-width products);
* "e3m2"      E3M2 P~ over E2M3 operands (two FP6 element formats);
* "affine"    E2M1 codes by one affine rule (EFQ-style);
* "exact_exp" the exact exponential in place of the bit pattern.

Parity bar as for the default map: relative L2 <= 2e-3 beyond what the
kernel's fp32 exponent placement can move near-tie codes, frozen max to fp32
rounding, fallback offsets exact outside the borderline rows.  The error
criterion (fused <= 1.1 x exp-then-quantize against exact attention, per
head) is asserted for the variants that meet it on the oracle; for "row"
and "affine" the oracle itself exceeds it on some heads (one E4M3 scale
flushes the tail of high-gain rows; the affine rule flushes values below
0.59 of a binade), so their ratios are printed and held to that accuracy.
"""

import concurrent.futures
import os

import numpy as np
import pytest

import workloads as W
import oracle as O
from oracle import FORMATS
from oracle.attention import mitchell_exp2
from gpu_helpers import (announce, to_dev, from_dev_bf16, rel_l2, workload_tensors, check_kappa,
                         kappa_borderline, check_frozen_max, kappa_free, kappa_rows,
                         kappa_low)
from parity import excess_rel_l2, eps_rows, kappa_eps, undecided

pytestmark = pytest.mark.gpu
TOL = 2e-3

# name, operand formats, oracle keywords, P~ format, oracle mode
VARIANTS = [
    ("row", "e4m3", dict(p_mode="row"), "e4m3", "row"),
    ("e4m3", "e2m3", dict(p_fmt="e4m3"), "e4m3", "block"),
    ("e4m3", "e2m1", dict(p_fmt="e4m3"), "e4m3", "block"),
    ("e3m2", "e2m3", dict(p_fmt="e3m2"), "e3m2", "block"),
    ("affine", "e2m1", dict(p_mode="efq"), "e2m1", "efq"),
    ("exact_exp", "e4m3", dict(p_mode="exp"), "e4m3", "exp"),
    ("exact_exp", "e2m3", dict(p_mode="exp"), "e2m3", "exp"),
    ("exact_exp", "e2m1", dict(p_mode="exp"), "e2m1", "exp"),
]
IDS = ["%s-%s" % (v[0], v[1]) for v in VARIANTS]


def _run(q, k, v, fmt, variant, causal=False, **kw):
    import torch
    import softmax_mx_quantize_amd as fsa
    out, kap, mg = fsa.attention_fwd(to_dev(q), to_dev(k), to_dev(v), fmt, causal, return_rows=True,
                                     p_variant=variant, **kw)
    torch.cuda.synchronize()
    return from_dev_bf16(out), kap.cpu().numpy(), mg.cpu().numpy()


def _borderline(info, rows, S, causal, fmt, pfmt, mode):
    """Rows whose kappa may differ by one: near a whole-binade step of the
    top block (all variants), and for one scale per row also near the
    overflow threshold that decides whether the row falls back at all."""
    eps = kappa_eps(info, fmt)
    border = kappa_borderline(info["scores"], info["m_tilde"], rows, S, causal, FORMATS[pfmt].mbits, eps,
                              exact=(mode == "exp"), low=kappa_low(pfmt, mode))
    if mode == "row":
        j = np.arange(S)[None, :]
        vis = (j <= np.asarray(rows)[:, None]) if causal else np.ones((len(rows), S), bool)
        tmax = np.where(vis, info["scores"] - info["m_tilde"][:, None], -np.inf).max(axis=1)
        # the score whose Mitchell value at the placement reaches the threshold
        thr = O.attention.overflow_threshold(pfmt)
        e = np.floor(np.log2(thr))
        t_over = e + thr / 2.0 ** e - 1.0 - O.attention.placement_exponent(pfmt)
        border |= np.abs(tmax - t_over) < eps
    return kappa_rows(border, kappa_free(info, pfmt, mode, eps), eps)


def _check(g, kap, mg, q, k, v, fmt, okw, pfmt, mode, causal=False, rows=None, bias=0.0):
    B, H, S, D = g.shape
    num = den = 0.0
    for b in range(B):
        for h in range(H):
            qh, kh, vh = (W.bf16_bits_to_f64(x[b, h]) for x in (q, k, v))
            ref, info = O.fused_attention(qh, kh, vh, fmt, causal, rows=rows, bias=bias,
                                          return_info=True, **okw)
            rws = np.arange(S) if rows is None else np.asarray(rows)
            gr, kr, mr = g[b, h, rws], kap[b, h, rws], mg[b, h, rws]
            check_frozen_max(mr, info, fmt)
            codes = _borderline(info, rws, S, causal, fmt, pfmt, mode)
            ex, _ = excess_rel_l2(gr, ref, info, pfmt, eps_rows(mr, info, fmt), mode,
                                  skip=undecided(codes, kr, info["kappa"]))
            num += (ex * np.linalg.norm(ref)) ** 2
            den += np.linalg.norm(ref) ** 2
            check_kappa(kr, info["kappa"], codes)
    err = float(np.sqrt(num / den))
    print("beyond near-tie codes %.2e" % err)
    assert err <= TOL, err


@pytest.mark.parametrize("variant", VARIANTS, ids=IDS)
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_variant_small_ragged(variant, D, causal):
    name, fmt, okw, pfmt, mode = variant
    S = 333
    announce("variant small", name, fmt, D, causal)
    q, k, v = (W.random_bf16((2, 2, S, D), seed, 1.3) for seed in (81, 82, 83))
    g, kap, mg = _run(q, k, v, fmt, name, causal)
    _check(g, kap, mg, q, k, v, fmt, okw, pfmt, mode, causal)


@pytest.mark.parametrize("variant", VARIANTS, ids=IDS)
def test_variant_fallbacks(variant):
    """Every row above its guess: by a few binades (in-sweep shifts, or the
    re-based pass for one scale per row) and by ~100 binades (re-based)."""
    name, fmt, okw, pfmt, mode = variant
    announce("variant fallback", name, fmt)
    q, k, v = (W.random_bf16((1, 2, 400, 128), seed, 1.0) for seed in (84, 85, 86))
    for bias in (-8.0, -100.0):
        g, kap, mg = _run(q, k, v, fmt, name, guess_bias=bias)
        assert np.all(kap > 0)
        _check(g, kap, mg, q, k, v, fmt, okw, pfmt, mode, bias=bias)


# guesses far above every row: 32 binades flush every code under one E4M3
# scale per row; 160 binades exceed what the largest block shift can reach
FAR_ABOVE = ([("row", "e4m3", dict(p_mode="row"), "e4m3", "row", 32.0)] +
             [("block", f, {}, f, "block", 160.0) for f in ("e4m3", "e2m3", "e2m1")] +
             [v + (160.0,) for v in VARIANTS if v[0] != "row"])


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", FAR_ABOVE, ids=["%s-%s" % c[:2] for c in FAR_ABOVE])
def test_guess_far_above_rows_fall_back(case, causal):
    """With the guess far above every row, each code would flush to zero (a
    zero row sum, 0/0 out); the rows fall back and are re-based downwards by
    their own top binade (negative kappa)."""
    name, fmt, okw, pfmt, mode, bias = case
    announce("guess far above", name, fmt, bias, causal)
    q, k, v = (W.random_bf16((1, 2, 333, 128), seed, 1.0) for seed in (94, 95, 96))
    g, kap, mg = _run(q, k, v, fmt, name, causal, guess_bias=bias)
    assert np.all(np.isfinite(g)) and np.all(kap < 0)
    _check(g, kap, mg, q, k, v, fmt, okw, pfmt, mode, causal, bias=bias)


# 230 binades: past 127 + REF = 189, where the scores' bit patterns
# themselves turn negative, so that the fallback pass measures the rows'
# offsets below zero
FAR_BELOW = ([("row", "e4m3", dict(p_mode="row"), "e4m3", "row")] +
             [("block", f, {}, f, "block") for f in ("e4m3", "e2m3", "e2m1")] +
             [v for v in VARIANTS if v[0] != "row"])


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", FAR_BELOW, ids=["%s-%s" % c[:2] for c in FAR_BELOW])
def test_guess_230_binades_above_rows(case, causal):
    """Rows about 230 binades below their guess (the largest bias the
    library takes is 240): each is re-based downwards by its own top binade,
    with kappa a few binades below -230 (the frozen max's spread term can
    lie a little above the row's top score)."""
    name, fmt, okw, pfmt, mode = case
    bias = 230.0
    announce("guess 230 above", name, fmt, causal)
    q, k, v = (W.random_bf16((1, 2, 333, 128), seed, 1.0) for seed in (111, 112, 113))
    g, kap, mg = _run(q, k, v, fmt, name, causal, guess_bias=bias)
    assert np.all(np.isfinite(g)) and np.all(kap <= -200) and np.all(kap >= -240)
    _check(g, kap, mg, q, k, v, fmt, okw, pfmt, mode, causal, bias=bias)


@pytest.mark.parametrize("variant", VARIANTS, ids=IDS)
def test_variant_clustered_keys(variant):
    """Two opposite key clusters: under the capped guess (64 binades above
    the window max) no row of a block map falls back, while one scale per
    row flushes such rows and re-bases them downwards; raised by a bias of
    150 binades, every row lies beyond 189 binades below its guess and is
    re-based downwards in every map."""
    name, fmt, okw, pfmt, mode = variant
    announce("variant clustered keys", name, fmt)
    q, k, v = W.two_valued_keys(1, 2, 600, 128, seed=42)
    for causal in (False, True):
        g, kap, mg = _run(q, k, v, fmt, name, causal)
        assert np.all(np.isfinite(g)) and np.all(kap >= -65) and (mode == "row" or np.all(kap == 0))
        _check(g, kap, mg, q, k, v, fmt, okw, pfmt, mode, causal)
        g, kap, mg = _run(q, k, v, fmt, name, causal, guess_bias=150.0)
        assert np.all(np.isfinite(g)) and (kap < -189).any()
        _check(g, kap, mg, q, k, v, fmt, okw, pfmt, mode, causal, bias=150.0)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m3", "e2m1"])
def test_guess_at_the_low_threshold(fmt):
    """Guesses about 127 - pl binades above the rows, so that their top
    blocks straddle the largest shift: rows below it are re-based downwards,
    rows above it keep kappa = 0 and a clamped-free scale; the kernel and
    the oracle agree row by row (rows within the margin of the threshold
    itself left free)."""
    pl = O.attention.placement_exponent(FORMATS[fmt])
    bias = (127 - pl) - 1.5
    announce("guess at the low threshold", fmt, bias)
    q, k, v = (W.random_bf16((1, 2, 600, 128), seed, 1.0) for seed in (97, 98, 99))
    g, kap, mg = _run(q, k, v, fmt, "block", guess_bias=bias)
    assert np.all(np.isfinite(g))
    assert (kap < 0).any() and (kap == 0).any()
    _check(g, kap, mg, q, k, v, fmt, {}, fmt, "block", bias=bias)


@pytest.mark.parametrize("variant", VARIANTS, ids=IDS)
def test_variant_v_ones(variant):
    import torch
    name, fmt, okw, pfmt, mode = variant
    announce("variant v=1", name, fmt)
    q, k = (W.random_bf16((1, 2, 300, 128), seed, 2.0) for seed in (87, 88))
    v = W.f32_to_bf16_bits(np.ones((1, 2, 300, 128), np.float32))
    for causal in (False, True):
        g, _, _ = _run(q, k, v, fmt, name, causal)
        assert np.array_equal(g, np.ones_like(g))


@pytest.mark.parametrize("lead", [66.5, 67.5, 100.5])
def test_row_scale_overflow_seen_past_the_pattern_top(lead):
    """One scale per row: a row whose only value past E4M3's range lies 66 or
    more binades above its guess.  Its pattern then reaches the top of fp32's
    exponent field (a NaN bit pattern at 66, the sign bit from 67 on), where
    the converted code need not show the overflow; the row must still fall
    back.  One score of row 5 is planted 300 binades above the rest and the
    bias chosen from the oracle's scores so that it lands ``lead`` binades
    above the guess, every other value of the row far below."""
    import oracle.attention as OA
    announce("row scale overflow past the pattern top", lead)
    S, D = 200, 64
    q, k, v = (W.bf16_bits_to_f64(W.random_bf16((1, 1, S, D), seed, 0.3)) for seed in (151, 152, 153))
    c = OA.score_scale(D)
    i, j = 5, 150
    q[0, 0, i] = k[0, 0, j] * (300.0 / (c * float(k[0, 0, j] @ k[0, 0, j])))
    q, k, v = (W.f32_to_bf16_bits(x.astype(np.float32)) for x in (q, k, v))
    qh, kh, vh = (W.bf16_bits_to_f64(x[0, 0]) for x in (q, k, v))
    _, info = O.fused_attention(qh, kh, vh, "e4m3", False, return_info=True, p_mode="row")
    t = np.sort(info["scores"][i] - info["m_tilde"][i])[::-1]
    bias = float(np.float32(t[0] - lead))
    assert t[0] - t[1] > lead + 2.0
    g, kap, mg = _run(q, k, v, "e4m3", "row", guess_bias=bias)
    _, info = O.fused_attention(qh, kh, vh, "e4m3", False, return_info=True, p_mode="row", bias=bias)
    assert info["kappa"][i] >= 66 and kap[0, 0, i] == info["kappa"][i]
    _check(g, kap, mg, q, k, v, "e4m3", dict(p_mode="row"), "e4m3", "row", bias=bias)


def test_variant_rejects_unbuilt_formats():
    import torch
    import softmax_mx_quantize_amd as fsa
    q = torch.zeros((1, 2, 64, 128), dtype=torch.bfloat16, device="cuda")
    for variant, fmt in (("row", "e2m1"), ("affine", "e4m3"), ("e4m3", "e4m3"), ("e3m2", "e2m1"),
                         ("e3m2", "e4m3")):
        with pytest.raises(fsa.FsaError) as e:
            fsa.attention_fwd(q, q, q, fmt, p_variant=variant)
        assert e.value.status == -2
    # the exact exponential over FP8 heads mixed with FP6/FP4 ones is not built
    with pytest.raises(fsa.FsaError) as e:
        fsa.attention_fwd(q, q, q, "e4m3", p_variant="exact_exp", head_fmt=["e4m3", "e2m1"])
    assert e.value.status == -2


def _threads():
    try:
        n = len(os.sched_getaffinity(0))
    except Exception:
        n = os.cpu_count() or 4
    return max(1, min(16, n))


# full-size variants: Video-DiT tensors, each variant's own formats
FULL = [("row", "e4m3"), ("e4m3", "e2m3"), ("e4m3", "e2m1"), ("e3m2", "e2m3"), ("affine", "e2m1"),
        ("exact_exp", "e4m3"), ("exact_exp", "e2m3"), ("exact_exp", "e2m1")]
CRIT_MET = {"e4m3", "e3m2", "exact_exp"}
# variants whose definition misses the 1.1 bar on some heads (host runs of
# the oracle: up to ~1.4 for one E4M3 scale per row, ~1.5 for the affine
# E2M1 codes): a looser bound that still catches a broken kernel
CRIT_ORACLE = {("row", "e4m3"): 2.0, ("affine", "e2m1"): 2.0}


@pytest.mark.parametrize("name,fmt", FULL, ids=["%s-%s" % f for f in FULL])
def test_variant_full_size(name, fmt):
    """One row of every query tile of two heads against the oracle, then the
    error criterion on every head (256 rows each)."""
    import torch
    import softmax_mx_quantize_amd as fsa
    variant = [v for v in VARIANTS if v[0] == name and v[1] == fmt][0]
    _, _, okw, pfmt, mode = variant
    w = W.WORKLOADS["video_dit_e4m3"]
    announce("variant full size", name, fmt)
    q, k, v = workload_tensors(w)
    out, kap, mg = fsa.attention_fwd(to_dev(q), to_dev(k), to_dev(v), fmt, False, return_rows=True,
                                     p_variant=name)
    torch.cuda.synchronize()
    g = from_dev_bf16(out)
    kap = kap.cpu().numpy()
    mg = mg.cpu().numpy()
    del out
    n_q = w.S // 128
    for h in (0, 23):
        rows = np.arange(n_q) * 128 + (np.arange(n_q) * 37 + h) % 128
        qh, kh, vh = (W.bf16_bits_to_f64(x[0, h]) for x in (q, k, v))
        ref, info = O.fused_attention(qh, kh, vh, fmt, False, rows=rows, return_info=True, **okw)
        codes = _borderline(info, rows, w.S, False, fmt, pfmt, mode)
        ex, n_allow = excess_rel_l2(g[0, h, rows], ref, info, pfmt, eps_rows(mg[0, h, rows], info, fmt), mode,
                                    skip=undecided(codes, kap[0, h, rows], info["kappa"]))
        print("%s-%s head %d: rel L2 %.2e, beyond near-tie codes %.2e" % (name, fmt, h, rel_l2(g[0, h, rows], ref), ex))
        assert ex <= TOL, (h, ex)
        check_kappa(kap[0, h, rows], info["kappa"], codes)

    def errs(h):
        rows = np.sort(np.random.default_rng([91, h]).choice(w.S, 256, replace=False))
        qh, kh, vh = (W.bf16_bits_to_f64(x[0, h]) for x in (q, k, v))
        exa = O.exact_attention(qh, kh, vh, rows=rows)
        pl = O.plain_mx_attention(qh, kh, vh, fmt, rows=rows, p_fmt=pfmt)
        return (np.sum((g[0, h, rows] - exa) ** 2, axis=1), np.sum((pl - exa) ** 2, axis=1))

    with concurrent.futures.ThreadPoolExecutor(_threads()) as pool:
        res = list(pool.map(errs, range(w.H)))
    ratios = [float(np.sqrt(a.sum() / b.sum())) for a, b in res]
    pooled = float(np.sqrt(sum(a.sum() for a, _ in res) / sum(b.sum() for _, b in res)))
    print("%s-%s per-head ratios: %s; pooled %.3f" % (name, fmt, " ".join("%.3f" % r for r in ratios), pooled))
    if name in CRIT_MET:
        assert pooled <= 1.1
        assert max(ratios) <= 1.1 + 0.02, max(ratios)
    else:
        assert max(ratios) <= CRIT_ORACLE[(name, fmt)], max(ratios)
