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
rows up to rows whose scores spread over a hundred binades) in every map,
and another keys in two opposite clusters (the guess's extreme-value term
far above the rows and held by its cap; workloads.two_valued_keys), and
another the workload recipes' heavy-tailed keys and planted outliers; a
fourth passes each of q, k, v and out in its own layout (contiguous
[B, H, S, D], a [B, S, H, D] tensor viewed as [B, H, S, D], or rows padded
to a longer stride); a fifth compares the allocation-free entry point with
the allocating one bit for bit; a sixth draws long sequences (2,000 to
20,000 keys) and checks sampled rows, the first and last among them.  Two
more cover the public MX quantiser (random ragged shapes, per-row binade
spreads, both block axes: bit for bit) and the BF16 baseline (random shapes
against exact attention); a last one checks the attention path's own
operands (Q'^ from the prologue, K^ and V^T with their tile-ordered scales)
bit for bit over random shapes.  A wide sweep reruns the shape, variant,
extreme and clustered generators with five more seeds (1,600 cases).
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


def _cluster_cases(n=24, seed=2031):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        var = MAPS[int(rng.integers(0, len(MAPS)))]
        H = int(rng.integers(1, 3))
        S = int(rng.integers(1, 901))
        D = int(rng.choice([64, 128]))
        causal = bool(rng.integers(0, 2))
        a = float(rng.uniform(0.3, 2.5))
        period = int(rng.choice([2, 3, 8, 32]))
        noise = float(rng.choice([0.05, 0.3, 1.0]))
        bias = float(rng.choice([0.0, 0.0, -8.0, 32.0, 150.0]))
        out.append((i, var, H, S, D, causal, a, period, noise, bias))
    return out


TCASES = _cluster_cases()


def _tid(c):
    i, var, H, S, D, causal, a, period, noise, bias = c
    return "t%02d-%s-%s-H%dS%dD%d%s-a%.2f-p%d-n%g-b%g" % (i, var[0], var[1], H, S, D,
                                                         "-causal" if causal else "", a, period,
                                                         noise, bias)


@pytest.mark.parametrize("case", TCASES, ids=[_tid(c) for c in TCASES])
def test_clustered_keys_all_rows(case):
    """Keys in two opposite clusters (one in ``period`` high): the guess's
    extreme-value term far above the rows, held by its cap to 64 binades
    above the window max; with a bias of 150, rows beyond 189 binades below
    their guess."""
    i, (name, fmt, okw, pfmt, mode), H, S, D, causal, a, period, noise, bias = case
    announce("fsa clustered-keys sweep", _tid(case))
    q, k, v = W.two_valued_keys(1, H, S, D, seed=1700 + i, a=a, gain=(0.2, 2.0), noise=noise,
                                period=period)
    g, kap, mg = _vrun(q, k, v, fmt, name, causal, guess_bias=bias)
    _vcheck(g, kap, mg, q, k, v, fmt, okw, pfmt, mode, causal, bias=bias)


def _heavy_cases(n=24, seed=2033):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        H = int(rng.integers(1, 4))
        S = int(rng.integers(100, 1501))
        D = int(rng.choice([64, 128]))
        causal = bool(rng.integers(0, 2))
        fmts = tuple(FMTS[int(j)] for j in rng.integers(0, 3, size=H))
        w = W.Workload("heavy", 1, H, S, D, causal, int(rng.integers(0, 1 << 30)), fmts,
                       gain_range=(float(rng.uniform(0.3, 1.0)), float(rng.uniform(1.0, 3.0))),
                       outlier_frac=float(rng.choice([0.0, 0.02, 0.1])),
                       outlier_sigma=float(rng.choice([8.0, 20.0, 60.0])),
                       heavy_frac=float(rng.choice([0.0, 0.05, 0.3])),
                       heavy_nu=float(rng.choice([1.5, 2.5, 4.0])))
        out.append((i, w))
    return out


HCASES = _heavy_cases()


def _hid(c):
    i, w = c
    return "h%02d-H%dS%dD%d%s-%s-out%g@%g-heavy%g@nu%g" % (
        i, w.H, w.S, w.D, "-causal" if w.causal else "", "+".join(w.head_fmts), w.outlier_frac,
        w.outlier_sigma, w.heavy_frac, w.heavy_nu)


@pytest.mark.parametrize("case", HCASES, ids=[_hid(c) for c in HCASES])
def test_heavy_tails_and_outliers_all_rows(case):
    """The workload recipes' heavy-tailed keys (Student-t down to 1.5 degrees
    of freedom: scores thousands of binades apart) and planted outlier scores
    (8 to 60 sigma), at small sizes, per-head formats in one launch."""
    i, w = case
    announce("fsa heavy-tail sweep", _hid(case))
    q, k, v = W.generate(w)
    g, kap, mg = _run(q, k, v, w.head_fmts[0], w.causal, head_fmt=list(w.head_fmts))
    _check(g, kap, mg, *_oracle_heads(q, k, v, list(w.head_fmts), w.causal))


LAYOUTS = ["bhsd", "bshd", "pad8", "pad16"]


def _layout_cases(n=24, seed=2027):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        B = int(rng.integers(1, 3))
        H = int(rng.integers(1, 5))
        S = int(rng.integers(1, 401))
        D = int(rng.choice([64, 128]))
        causal = bool(rng.integers(0, 2))
        fmts = tuple(FMTS[int(j)] for j in rng.integers(0, 3, size=H))
        lay = tuple(LAYOUTS[int(j)] for j in rng.integers(0, len(LAYOUTS), size=4))
        out.append((i, B, H, S, D, causal, fmts, lay))
    return out


LCASES = _layout_cases()


def _lid(c):
    i, B, H, S, D, causal, fmts, lay = c
    return "l%02d-B%dH%dS%dD%d%s-%s-%s" % (i, B, H, S, D, "-causal" if causal else "", "+".join(fmts),
                                          "/".join(lay))


def _view(x, lay):
    """A [B, H, S, D] bf16 device view of the host bits ``x`` (None: an
    uninitialised output) stored in layout ``lay``."""
    import torch
    from gpu_helpers import to_dev
    B, H, S, D = x.shape
    if lay == "bhsd":
        return to_dev(x)
    if lay == "bshd":
        return to_dev(np.ascontiguousarray(x.transpose(0, 2, 1, 3))).transpose(1, 2)
    pad = int(lay[3:])
    store = torch.zeros((B, H, S, D + pad), dtype=torch.bfloat16, device="cuda")
    store[..., :D] = to_dev(x)
    return store[..., :D]


@pytest.mark.parametrize("case", LCASES, ids=[_lid(c) for c in LCASES])
def test_strided_layouts_all_rows(case):
    import torch
    import softmax_mx_quantize_amd as fsa
    from gpu_helpers import from_dev_bf16
    i, B, H, S, D, causal, fmts, lay = case
    announce("fsa layout sweep", _lid(case))
    q, k, v = (W.random_bf16((B, H, S, D), 1700 + 3 * i + j, 1.2) for j in range(3))
    dq, dk, dv = (_view(x, l) for x, l in zip((q, k, v), lay))
    out = _view(np.zeros((B, H, S, D), np.uint16), lay[3])
    o, kap, mg = fsa.attention_fwd(dq, dk, dv, fmts[0], causal, head_fmt=list(fmts), out=out,
                                   return_rows=True)
    torch.cuda.synchronize()
    assert o.data_ptr() == out.data_ptr()
    g = from_dev_bf16(o.contiguous())
    _check(g, kap.cpu().numpy(), mg.cpu().numpy(), *_oracle_heads(q, k, v, list(fmts), causal))
    # the views change addressing only: the contiguous call gives the same bits
    from gpu_helpers import to_dev
    oc, kc, mc = fsa.attention_fwd(to_dev(q), to_dev(k), to_dev(v), fmts[0], causal, head_fmt=list(fmts),
                                   return_rows=True)
    torch.cuda.synchronize()
    gc = from_dev_bf16(oc)
    assert np.array_equal(g, gc) or np.array_equal(np.isnan(g), np.isnan(gc)) and np.array_equal(
        np.nan_to_num(g), np.nan_to_num(gc))
    assert np.array_equal(kap.cpu().numpy(), kc.cpu().numpy()) and np.array_equal(mg.cpu().numpy(), mc.cpu().numpy())


def _noalloc_cases(n=24, seed=2028):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        B = int(rng.integers(1, 3))
        H = int(rng.integers(1, 5))
        S = int(rng.integers(1, 3001))
        D = int(rng.choice([64, 128]))
        causal = bool(rng.integers(0, 2))
        fmts = tuple(FMTS[int(j)] for j in rng.integers(0, 3, size=H))
        bias = float(rng.choice([0.0, 0.0, -8.0, -100.0, 150.0]))
        variant = str(rng.choice(["block", "block", "exact_exp"]))
        if variant == "exact_exp" and "e4m3" in fmts and len(set(fmts)) > 1:
            # built for one format per call or the FP6/FP4 hybrid
            fmts = tuple("e2m3" if f == "e4m3" else f for f in fmts)
        out.append((i, B, H, S, D, causal, fmts, bias, variant))
    return out


NCASES = _noalloc_cases()


def _nid(c):
    i, B, H, S, D, causal, fmts, bias, variant = c
    return "n%02d-B%dH%dS%dD%d%s-%s-b%g-%s" % (i, B, H, S, D, "-causal" if causal else "",
                                               "+".join(fmts), bias, variant)


@pytest.mark.parametrize("case", NCASES, ids=[_nid(c) for c in NCASES])
def test_noalloc_matches_allocating_call(case):
    """The allocation-free entry point runs the same kernels on the same
    inputs: outputs, fallback offsets and frozen maxima bit for bit."""
    import torch
    import softmax_mx_quantize_amd as fsa
    from gpu_helpers import to_dev
    i, B, H, S, D, causal, fmts, bias, variant = case
    announce("fsa no-alloc sweep", _nid(case))
    q, k, v = (to_dev(W.random_bf16((B, H, S, D), 1900 + 3 * i + j, 1.2)) for j in range(3))
    kw = dict(head_fmt=list(fmts), guess_bias=bias, p_variant=variant, return_rows=True)
    a = fsa.attention_fwd(q, k, v, fmts[0], causal, **kw)
    b = fsa.attention_fwd(q, k, v, fmts[0], causal, no_alloc=True, **kw)
    torch.cuda.synchronize()
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
    assert torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])


def _long_cases(n=12, seed=2029):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        B = int(rng.integers(1, 3))
        H = int(rng.integers(1, 4))
        S = int(rng.integers(2000, 20001))
        D = int(rng.choice([64, 128]))
        causal = bool(rng.integers(0, 2))
        fmts = tuple(FMTS[int(j)] for j in rng.integers(0, 3, size=H))
        scale = float(rng.uniform(0.5, 2.0))
        bias = float(rng.choice([0.0, 0.0, -8.0, -100.0, 150.0]))
        rows = np.unique(np.concatenate([[0, S - 1], rng.integers(0, S, size=62)]))
        out.append((i, B, H, S, D, causal, fmts, scale, bias, rows))
    return out


GCASES = _long_cases()


def _gid(c):
    i, B, H, S, D, causal, fmts, scale, bias, rows = c
    return "g%02d-B%dH%dS%dD%d%s-%s-x%.1f-b%g" % (i, B, H, S, D, "-causal" if causal else "",
                                                  "+".join(fmts), scale, bias)


@pytest.mark.parametrize("case", GCASES, ids=[_gid(c) for c in GCASES])
def test_long_sequences_sampled_rows(case):
    i, B, H, S, D, causal, fmts, scale, bias, rows = case
    announce("fsa long sweep", _gid(case))
    q, k, v = (W.random_bf16((B, H, S, D), 2100 + 3 * i + j, scale if j < 2 else 1.0)
               for j in range(3))
    g, kap, mg = _run(q, k, v, fmts[0], causal, head_fmt=list(fmts), guess_bias=bias)
    ref, rk, bd, inf = _oracle_heads(q, k, v, list(fmts), causal, rows=rows, bias=bias)
    _check(g, kap, mg, ref.reshape(B * H, len(rows), D), rk, bd, inf, rows=rows)


def _quant_cases(n=36, seed=2030):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        shape = (int(rng.integers(1, 4)), int(rng.integers(1, 400)), int(rng.integers(1, 400)))
        fmt = FMTS[int(rng.integers(0, 3))]
        along = int(rng.integers(0, 2))
        spread = int(rng.choice([0, 8, 40]))
        out.append((i, shape, fmt, along, spread))
    return out


QCASES = _quant_cases()


@pytest.mark.parametrize("case", QCASES, ids=["q%02d-%dx%dx%d-%s-rows%d-e%d" % ((c[0],) + c[1] + c[2:])
                                              for c in QCASES])
def test_quantizer_shapes_bit_exact(case):
    from test_gpu_quant import _gpu_quant, _oracle
    i, shape, fmt, along, spread = case
    announce("quant sweep", case)
    rng = np.random.default_rng(2300 + i)
    # blocks at binades spread over +-spread (along the blocks' axis: per element)
    e = rng.integers(-spread, spread + 1, size=shape) if spread else 0
    x = (rng.standard_normal(shape) * np.exp2(e)).astype(np.float32)
    bits = W.f32_to_bf16_bits(x)
    gc, gs = _gpu_quant(bits, fmt, along)
    oc, os_ = _oracle(bits, fmt, along)
    assert np.array_equal(gs, os_)
    assert np.array_equal(gc, oc)


def _bf16_cases(n=16, seed=2031):
    rng = np.random.default_rng(seed)
    return [(i, int(rng.integers(1, 3)), int(rng.integers(1, 4)), int(rng.integers(1, 1500)),
             int(rng.choice([64, 128])), bool(rng.integers(0, 2)), float(rng.uniform(0.5, 2.5)))
            for i in range(n)]


BCASES = _bf16_cases()


@pytest.mark.parametrize("case", BCASES, ids=["b%02d-B%dH%dS%dD%d-c%d-x%.1f" % (c[0], c[1], c[2], c[3], c[4],
                                                                              c[5], c[6]) for c in BCASES])
def test_bf16_baseline_shapes(case):
    import oracle as O
    from test_gpu_bf16 import _run as _brun, TOL as BTOL
    from gpu_helpers import rel_l2
    i, B, H, S, D, causal, scale = case
    announce("bf16 sweep", case)
    q, k, v = (W.random_bf16((B, H, S, D), 2500 + 3 * i + j, scale if j < 2 else 1.0) for j in range(3))
    g = _brun(q, k, v, causal)
    for b in range(B):
        for h in range(H):
            qh, kh, vh = (W.bf16_bits_to_f64(x[b, h]) for x in (q, k, v))
            ex = O.exact_attention(qh, kh, vh, causal)
            assert rel_l2(g[b, h], ex) <= BTOL, (b, h)


def _operand_cases(n=16, seed=2032):
    rng = np.random.default_rng(seed)
    return [(i, int(rng.integers(1, 3)), int(rng.integers(1, 3)), int(rng.integers(1, 900)),
             int(rng.choice([64, 128])), FMTS[int(rng.integers(0, 3))], int(rng.choice([0, 6, 30])))
            for i in range(n)]


OCASES = _operand_cases()


@pytest.mark.parametrize("case", OCASES, ids=["o%02d-B%dH%dS%dD%d-%s-e%d" % c for c in OCASES])
def test_operands_shapes_bit_exact(case):
    import torch
    import softmax_mx_quantize_amd as fsa
    from gpu_helpers import to_dev
    from test_gpu_operands import _check_head
    i, B, H, S, D, fmt, spread = case
    announce("operands sweep", case)
    rng = np.random.default_rng(2600 + i)
    xs = []
    for j in range(3):
        e = rng.integers(-spread, spread + 1, size=(B, H, S, 1)) if spread else 0
        xs.append(W.f32_to_bf16_bits((rng.standard_normal((B, H, S, D)) * np.exp2(e)).astype(np.float32)))
    q, k, v = xs
    got = fsa.debug_operands(to_dev(q), to_dev(k), to_dev(v), fmt)
    torch.cuda.synchronize()
    for b in range(B):
        for h in range(H):
            _check_head(got, *(W.bf16_bits_to_f64(x[b, h]) for x in (q, k, v)), fmt, b, h)


# Wider runs of the same generators: five more seeds, each generator's cases
# run in one test item (so that a failure names every case that failed).
WIDE_SEEDS = [7000, 9000, 11000, 13000, 15000]
WIDE = [("mixed", lambda sd: _cases(n=120, seed=sd), test_mixed_shapes_all_rows, _id),
        ("variants", lambda sd: _variant_cases(per=10, seed=sd + 1), test_variant_mixed_shapes_all_rows, _vid),
        ("extreme", lambda sd: _extreme_cases(n=60, seed=sd + 2), test_extreme_score_spreads_all_rows, _xid),
        ("clustered", lambda sd: _cluster_cases(n=60, seed=sd + 3), test_clustered_keys_all_rows, _tid)]


@pytest.mark.parametrize("seed", WIDE_SEEDS)
@pytest.mark.parametrize("gen", WIDE, ids=[g[0] for g in WIDE])
def test_wide_sweep(gen, seed):
    name, make, run, idf = gen
    failed = []
    for c in make(seed):
        try:
            run(c)
        except AssertionError as e:
            failed.append((idf(c), str(e)[:120]))
    announce("wide sweep", name, seed, "failed:", len(failed))
    assert not failed, failed
