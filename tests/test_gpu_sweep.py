"""A seeded sweep of mixed call shapes against the float64 oracle, all rows.

Each case draws B in {1, 2}, H in {1, 2, 3} (per-head formats drawn
independently, so most multi-head cases are hybrid launches), S in [1, 700]
(ragged key and query tiles), D in {64, 128}, causal or not, an input scale
(score spread) and a frozen-max bias: 0, a lowered guess that sends rows
through the in-sweep shifts (-8 binades) or the second pass (-100), or a
raised one (32: one E4M3 scale per row flushes; 150: every map flushes),
whose rows are re-based downwards.  The
bar is the one of the other parity tests (tests/parity.py).  A second sweep
draws the same kinds of shapes for each P~ variant (one format per call); a
third draws extreme score spreads (input scales 0.05 to 6: nearly uniform
rows up to rows whose scores spread over a hundred binades) in every map.
"""

import numpy as np
import pytest

import workloads as W
from gpu_helpers import announce
from test_gpu_fsa import _run, _oracle_heads, _check
from test_gpu_variants import VARIANTS, _run as _vrun, _check as _vcheck

pytestmark = pytest.mark.gpu
FMTS = ["e4m3", "e2m3", "e2m1"]


def _cases(n=48, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        B = int(rng.integers(1, 3))
        H = int(rng.integers(1, 4))
        S = int(rng.integers(1, 701))
        D = int(rng.choice([64, 128]))
        causal = bool(rng.integers(0, 2))
        fmts = [FMTS[int(j)] for j in rng.integers(0, 3, size=H)]
        scale = float(rng.uniform(0.5, 2.5))
        bias = float(rng.choice([0.0, 0.0, -8.0, -100.0, 32.0, 150.0]))
        out.append((i, B, H, S, D, causal, tuple(fmts), scale, bias))
    return out


CASES = _cases()


def _id(c):
    i, B, H, S, D, causal, fmts, scale, bias = c
    return "c%02d-B%dH%dS%dD%d%s-%s-x%.1f-b%g" % (i, B, H, S, D, "-causal" if causal else "",
                                                   "+".join(fmts), scale, bias)


@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
def test_mixed_shapes_all_rows(case):
    i, B, H, S, D, causal, fmts, scale, bias = case
    announce("fsa sweep", _id(case))
    q, k, v = (W.random_bf16((B, H, S, D), 500 + 3 * i + j, scale if j < 2 else 1.0)
               for j in range(3))
    g, kap, mg = _run(q, k, v, fmts[0], causal, head_fmt=list(fmts), guess_bias=bias)
    _check(g, kap, mg, *_oracle_heads(q, k, v, list(fmts), causal, bias=bias))


def _variant_cases(per=4, seed=2025):
    rng = np.random.default_rng(seed)
    out = []
    for vi, var in enumerate(VARIANTS):
        for r in range(per):
            B = int(rng.integers(1, 3))
            H = int(rng.integers(1, 3))
            S = int(rng.integers(1, 601))
            D = int(rng.choice([64, 128]))
            causal = bool(rng.integers(0, 2))
            scale = float(rng.uniform(0.5, 2.5))
            bias = float(rng.choice([0.0, 0.0, -8.0, -100.0, 32.0, 150.0]))
            out.append((vi * per + r, var, B, H, S, D, causal, scale, bias))
    return out


VCASES = _variant_cases()


def _vid(c):
    i, var, B, H, S, D, causal, scale, bias = c
    return "v%02d-%s-%s-B%dH%dS%dD%d%s-x%.1f-b%g" % (i, var[0], var[1], B, H, S, D,
                                                    "-causal" if causal else "", scale, bias)


@pytest.mark.parametrize("case", VCASES, ids=[_vid(c) for c in VCASES])
def test_variant_mixed_shapes_all_rows(case):
    i, (name, fmt, okw, pfmt, mode), B, H, S, D, causal, scale, bias = case
    announce("fsa variant sweep", _vid(case))
    q, k, v = (W.random_bf16((B, H, S, D), 900 + 3 * i + j, scale if j < 2 else 1.0)
               for j in range(3))
    g, kap, mg = _vrun(q, k, v, fmt, name, causal, guess_bias=bias)
    _vcheck(g, kap, mg, q, k, v, fmt, okw, pfmt, mode, causal, bias=bias)


MAPS = [("block", f, {}, f, "block") for f in FMTS] + VARIANTS


def _extreme_cases(n=24, seed=2026):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        var = MAPS[int(rng.integers(0, len(MAPS)))]
        S = int(rng.integers(1, 501))
        D = int(rng.choice([64, 128]))
        causal = bool(rng.integers(0, 2))
        scale = float(rng.choice([0.05, 3.5, 5.0, 6.0]))
        bias = float(rng.choice([0.0, -8.0, -100.0]))
        out.append((i, var, S, D, causal, scale, bias))
    return out


XCASES = _extreme_cases()


def _xid(c):
    i, var, S, D, causal, scale, bias = c
    return "x%02d-%s-%s-S%dD%d%s-x%.2f-b%g" % (i, var[0], var[1], S, D, "-causal" if causal else "",
                                               scale, bias)


@pytest.mark.parametrize("case", XCASES, ids=[_xid(c) for c in XCASES])
def test_extreme_score_spreads_all_rows(case):
    i, (name, fmt, okw, pfmt, mode), S, D, causal, scale, bias = case
    announce("fsa extreme sweep", _xid(case))
    q, k, v = (W.random_bf16((1, 1, S, D), 1300 + 3 * i + j, scale if j < 2 else 1.0)
               for j in range(3))
    g, kap, mg = _vrun(q, k, v, fmt, name, causal, guess_bias=bias)
    _vcheck(g, kap, mg, q, k, v, fmt, okw, pfmt, mode, causal, bias=bias)
