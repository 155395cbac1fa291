"""Exact properties of the fused path on the GPU, checked bit for bit against
the library's own output rather than the oracle:

* V scaled by a power of two: the MX blocks of V keep their codes and only
  their E8M0 scales move, P~ and the row sums do not depend on V, so the
  output scales by the same power exactly (while no value leaves bf16's
  normal range and the fp32 sums stay finite), also for rows shifted within
  the sweep or re-based by the fallback pass;
* Q scaled by 2^a and K by 2^-a: the codes stay, the block scales move in
  opposite directions, so every score and result stays the same;
* V's columns permuted: each output column is the product of P~ with one
  column of V (V is quantised along the keys, column by column), so the
  output's columns follow;
* query rows permuted (no causal mask): each row's frozen max, P~, offsets
  and sums depend on that row alone, so every row's results follow it
  wherever it sits in the tiles, with or without the fallback pass;
* a head placed anywhere in a larger call (other heads of other formats
  around it) gives the result it gives alone;
* with the causal mask, rows before a whole V block do not depend on the
  keys from that block on;
* with the causal mask, row i for i + 1 a multiple of 32 sees exactly the
  problem truncated to its first i + 1 keys (the same V blocks along the
  keys, the same frozen-max window), so it equals the last row of that
  problem without the mask.

Each of these would catch a misplaced scale, a row or column index that
depends on a tile position, or state shared between rows, heads or
formats, independently of the oracle's tolerance.
"""

import numpy as np
import pytest

import workloads as W
from gpu_helpers import announce
from test_gpu_fsa import _run
from test_gpu_variants import VARIANTS, _run as _vrun

pytestmark = pytest.mark.gpu
FMTS = ["e4m3", "e2m3", "e2m1"]
CASES = [("block", f) for f in FMTS] + [(v[0], v[1]) for v in VARIANTS]
IDS = ["%s-%s" % c for c in CASES]


def _call(q, k, v, name, fmt, causal=False, **kw):
    if name == "block":
        return _run(q, k, v, fmt, causal, **kw)
    return _vrun(q, k, v, fmt, name, causal, **kw)


def _scaled_bits(bits, k):
    """bf16 bits times 2^k (exact while the values stay normal)."""
    x = W.bf16_bits_to_f64(bits) * 2.0 ** k
    return W.f32_to_bf16_bits(x.astype(np.float32))


def _same(a, b):
    assert a.shape == b.shape
    bad = ~((a == b) | (np.isnan(a) & np.isnan(b)))
    assert not bad.any(), (int(bad.sum()), np.argwhere(bad)[:3])


@pytest.mark.parametrize("case", CASES, ids=IDS)
@pytest.mark.parametrize("causal", [False, True])
def test_v_scaled_by_a_power_of_two(case, causal):
    name, fmt = case
    announce("property: V * 2^k", name, fmt, causal)
    q, k, v = (W.random_bf16((1, 2, 333, 128), seed, 1.0) for seed in (121, 122, 123))
    vv = W.bf16_bits_to_f64(v)
    nz = vv[vv != 0]
    # every scaled value stays a normal bf16 number
    assert np.abs(nz).min() * 2.0 ** -100 >= 2.0 ** -126 and np.abs(vv).max() * 2.0 ** 100 < 2.0 ** 127
    g0, k0, m0 = _call(q, k, v, name, fmt, causal)
    for e in (-100, -37, 45, 100):
        g, kap, mg = _call(q, k, _scaled_bits(v, e), name, fmt, causal)
        _same(g, g0 * 2.0 ** e)
        assert np.array_equal(kap, k0) and np.array_equal(mg, m0)


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_v_scaled_through_the_fallbacks(case):
    """The same exactness for rows above their guess: by about 60 binades
    (their blocks take larger scales within the sweep, so the products sum
    P~ values near 2^60 before the division) and by about 100 (re-based by
    the fallback pass)."""
    name, fmt = case
    announce("property: V * 2^k, shifted rows", name, fmt)
    q, k, v = (W.random_bf16((1, 2, 333, 128), seed, 1.0) for seed in (141, 142, 143))
    for bias in (-60.0, -100.0):
        g0, k0, m0 = _call(q, k, v, name, fmt, guess_bias=bias)
        assert np.all(k0 >= 55)
        for e in (-60, 40):
            g, kap, mg = _call(q, k, _scaled_bits(v, e), name, fmt, guess_bias=bias)
            _same(g, g0 * 2.0 ** e)
            assert np.array_equal(kap, k0) and np.array_equal(mg, m0)


@pytest.mark.parametrize("case", CASES, ids=IDS)
@pytest.mark.parametrize("causal", [False, True])
def test_q_and_k_scaled_reciprocally(case, causal):
    """Q times 2^a and K times 2^-a: both keep their MX codes (Q's softmax
    scale is applied before its rounding, and a power of two commutes with
    it), their block scales move by a and -a, and every score, frozen max,
    offset and output stays the same bit for bit."""
    name, fmt = case
    announce("property: Q * 2^a, K * 2^-a", name, fmt, causal)
    q, k, v = (W.random_bf16((1, 2, 333, 128), seed, 1.0) for seed in (144, 145, 146))
    g0, k0, m0 = _call(q, k, v, name, fmt, causal)
    for a in (-40, 7, 40):
        g, kap, mg = _call(_scaled_bits(q, a), _scaled_bits(k, -a), v, name, fmt, causal)
        _same(g, g0)
        assert np.array_equal(kap, k0) and np.array_equal(mg, m0)


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_v_columns_permuted(case):
    name, fmt = case
    announce("property: V columns permuted", name, fmt)
    D = 128
    q, k, v = (W.random_bf16((1, 2, 300, D), seed, 1.0) for seed in (124, 125, 126))
    perm = np.random.default_rng(127).permutation(D)
    for causal in (False, True):
        g0, _, _ = _call(q, k, v, name, fmt, causal)
        g, _, _ = _call(q, k, np.ascontiguousarray(v[..., perm]), name, fmt, causal)
        _same(g, g0[..., perm])


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_query_rows_permuted(case):
    name, fmt = case
    announce("property: query rows permuted", name, fmt)
    S = 333
    q, k, v = (W.random_bf16((1, 2, S, 128), seed, 1.0) for seed in (128, 129, 130))
    perm = np.random.default_rng(131).permutation(S)
    qp = np.ascontiguousarray(q[:, :, perm])
    # as drawn, with every row sent through the fallback pass, and with every
    # row beyond the offsets the first pass records (measured again)
    for bias in (0.0, -100.0, -400.0):
        g0, k0, m0 = _call(q, k, v, name, fmt, guess_bias=bias)
        g, kap, mg = _call(qp, k, v, name, fmt, guess_bias=bias)
        _same(g, g0[:, :, perm])
        assert np.array_equal(kap, k0[:, :, perm]) and np.array_equal(mg, m0[:, :, perm])


def test_head_placed_in_a_larger_hybrid_call():
    announce("property: head placement")
    S, D = 300, 128
    fmts = ["e2m1", "e4m3", "e2m3"]
    # B = 2, H = 3, one format per head; each head against a call of its own
    q, k, v = (W.random_bf16((2, 3, S, D), seed, 1.0) for seed in (132, 133, 134))
    for causal in (False, True):
        g, kap, mg = _run(q, k, v, "e4m3", causal, head_fmt=fmts)
        for b in range(2):
            for h in range(3):
                one = tuple(np.ascontiguousarray(x[b:b + 1, h:h + 1]) for x in (q, k, v))
                g1, k1, m1 = _run(*one, fmts[h], causal)
                _same(g[b, h], g1[0, 0])
                assert np.array_equal(kap[b, h], k1[0, 0]) and np.array_equal(mg[b, h], m1[0, 0])


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_causal_rows_ignore_later_key_blocks(case):
    """With the causal mask, rows before key 160 (five whole 32-key blocks of
    V) cannot see keys 160 on: replacing those keys' K and V with far larger
    values leaves every such row's output, offset and frozen max unchanged,
    also with every row sent through the fallback pass."""
    name, fmt = case
    announce("property: causal rows ignore later keys", name, fmt)
    S, cut = 333, 160
    q, k, v = (W.random_bf16((1, 2, S, 128), seed, 1.0) for seed in (147, 148, 149))
    k2, v2 = (x.copy() for x in (k, v))
    k2[:, :, cut:] = W.random_bf16((1, 2, S - cut, 128), 150, 5.0)
    v2[:, :, cut:] = W.random_bf16((1, 2, S - cut, 128), 151, 50.0)
    for bias in (0.0, -100.0):
        g0, k0, m0 = _call(q, k, v, name, fmt, True, guess_bias=bias)
        g, kap, mg = _call(q, k2, v2, name, fmt, True, guess_bias=bias)
        _same(g[:, :, :cut], g0[:, :, :cut])
        assert np.array_equal(kap[:, :, :cut], k0[:, :, :cut])
        assert np.array_equal(mg[:, :, :cut], m0[:, :, :cut])
        assert not np.array_equal(g[:, :, cut:], g0[:, :, cut:])


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_causal_row_is_the_truncated_problem(case):
    name, fmt = case
    announce("property: causal row = truncated problem", name, fmt)
    S = 420
    q, k, v = (W.random_bf16((1, 1, S, 128), seed, 1.0) for seed in (135, 136, 137))
    g, kap, mg = _call(q, k, v, name, fmt, True)
    for i in (31, 127, 159, 255, 415):
        n = i + 1
        part = tuple(np.ascontiguousarray(x[:, :, :n]) for x in (q, k, v))
        gt, kt, mt = _call(*part, name, fmt, False)
        _same(g[0, 0, i], gt[0, 0, i])
        assert kap[0, 0, i] == kt[0, 0, i] and mg[0, 0, i] == mt[0, 0, i], i
