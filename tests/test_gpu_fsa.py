"""Fused-softmax attention on the GPU against the float64 oracle.

Bar: relative L2 <= 2e-3 against the oracle's fused result on the same
inputs, and on the small workload the error against exact attention stays
within 1.1x the exp-then-quantize error.  Fallback offsets agree row by row
(except rows within rounding of the overflow threshold, which are counted).
"""

import dataclasses

import numpy as np
import pytest

import workloads as W
import oracle as O
from gpu_helpers import (announce, to_dev, from_dev_bf16, rel_l2, kappa_borderline,
                         check_kappa, check_frozen_max, kappa_free, kappa_rows, kappa_low)
from oracle import FORMATS
from parity import excess_rel_l2, eps_rows, kappa_eps, undecided

pytestmark = pytest.mark.gpu
FMTS = ["e4m3", "e2m3", "e2m1"]
TOL = 2e-3


def _run(q, k, v, fmt, causal=False, **kw):
    import torch
    import softmax_mx_quantize_amd as fsa
    out, kap, mg = fsa.attention_fwd(to_dev(q), to_dev(k), to_dev(v), fmt, causal,
                                     return_rows=True, **kw)
    torch.cuda.synchronize()
    return from_dev_bf16(out), kap.cpu().numpy(), mg.cpu().numpy()


def _oracle_heads(q, k, v, fmts, causal=False, rows=None, bias=0.0):
    """The oracle per (batch, head): outputs, fallback offsets, borderline
    rows for kappa, and the info the tie allowance needs."""
    B, H, S = q.shape[:3]
    outs, kaps, borders, infos = [], [], [], []
    rws = np.arange(S) if rows is None else np.asarray(rows)
    for b in range(B):
        for h in range(H):
            qh, kh, vh = (W.bf16_bits_to_f64(x[b, h]) for x in (q, k, v))
            o, info = O.fused_attention(qh, kh, vh, fmts[h], causal, rows=rows, bias=bias,
                                        return_info=True)
            outs.append(o)
            kaps.append(info["kappa"])
            ke = kappa_eps(info, fmts[h])
            borders.append(kappa_rows(kappa_borderline(info["scores"], info["m_tilde"], rws, S, causal,
                                                       FORMATS[fmts[h]].mbits, ke,
                                                       low=kappa_low(fmts[h], "block")),
                                      kappa_free(info, fmts[h], "block", ke), ke))
            infos.append((info, fmts[h]))
    return np.stack(outs), np.stack(kaps), np.stack(borders), infos


def _check(gpu_out, gpu_kap, gpu_mg, ref_out, ref_kap, border, infos, rows=None):
    """Relative L2 against the oracle once the near-tie codes of the kernel's
    fp32 exponent placement are allowed either way (tests/parity.py), the
    frozen max to fp32 rounding, and the fallback offsets exactly outside
    the borderline rows."""
    B, H, S, D = gpu_out.shape
    g = gpu_out.reshape(B * H, S, D)
    kk = gpu_kap.reshape(B * H, S)
    mg = gpu_mg.reshape(B * H, S)
    if rows is not None:
        g = g[:, rows]
        kk = kk[:, rows]
        mg = mg[:, rows]
    num = 0.0
    for x in range(B * H):
        info, fmt = infos[x]
        check_frozen_max(mg[x], info, fmt)
        skip = undecided(border.reshape(B * H, -1)[x], kk[x], ref_kap.reshape(B * H, -1)[x])
        ex, _ = excess_rel_l2(g[x], ref_out[x], info, fmt, eps_rows(mg[x], info, fmt), skip=skip)
        num += (ex * np.linalg.norm(ref_out[x])) ** 2
    err = float(np.sqrt(num) / np.linalg.norm(ref_out))
    print("rel L2 %.2e, beyond near-tie codes %.2e" % (rel_l2(g, ref_out), err))
    assert err <= TOL, err
    check_kappa(kk.ravel(), ref_kap.ravel(), border.ravel())
    return err


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_small_ragged_all_rows(fmt, D, causal):
    S = 333                       # 3 key tiles, ragged; 3 query workgroups
    announce("fsa small", fmt, D, causal, S)
    q, k, v = (W.random_bf16((2, 2, S, D), seed, 1.3) for seed in (1, 2, 3))
    g, kap, mg = _run(q, k, v, fmt, causal)
    _check(g, kap, mg, *_oracle_heads(q, k, v, [fmt] * 2, causal))


@pytest.mark.parametrize("S", [1, 17, 128, 129, 640])
def test_edge_lengths(S):
    announce("fsa edge", S)
    for fmt in FMTS:
        for causal in (False, True):
            q, k, v = (W.random_bf16((1, 1, S, 128), seed, 1.0) for seed in (4, 5, 6))
            g, kap, mg = _run(q, k, v, fmt, causal)
            _check(g, kap, mg, *_oracle_heads(q, k, v, [fmt], causal))


@pytest.mark.parametrize("fmt", FMTS)
def test_v_ones_gives_exactly_one(fmt):
    announce("fsa v=1", fmt)
    q, k = (W.random_bf16((1, 2, 300, 128), seed, 2.0) for seed in (7, 8))
    v = W.f32_to_bf16_bits(np.ones((1, 2, 300, 128), np.float32))
    for causal in (False, True):
        g, _, _ = _run(q, k, v, fmt, causal)
        assert np.array_equal(g, np.ones_like(g))


@pytest.mark.parametrize("fmt", FMTS)
def test_forced_fallback_every_row(fmt):
    announce("fsa forced fallback", fmt)
    q, k, v = (W.random_bf16((1, 2, 400, 128), seed, 1.0) for seed in (9, 10, 11))
    g, kap, mg = _run(q, k, v, fmt, False, guess_bias=-8.0)
    assert np.all(kap > 0)
    _check(g, kap, mg, *_oracle_heads(q, k, v, [fmt] * 2, False, bias=-8.0))


@pytest.mark.parametrize("fmt", FMTS)
def test_rows_far_above_the_guess(fmt):
    """Rows whose scores exceed the frozen max by far more than the in-loop
    block shifts reach (64 binades) are recomputed with the re-based
    reference; their neighbours in the same wave must come out unchanged."""
    announce("fsa far fallback", fmt)
    S, D = 300, 128
    q, k, v = (W.bf16_bits_to_f64(W.random_bf16((1, 1, S, D), seed, 1.0)) for seed in (12, 13, 14))
    c = O.attention.score_scale(D)
    for i, j in ((5, 140), (77, 290), (200, 131)):
        # q_i along k_j, scaled so that this one score is ~300 binades
        q[0, 0, i] = k[0, 0, j] * (300.0 / (c * float(k[0, 0, j] @ k[0, 0, j])))
    q, k, v = (W.f32_to_bf16_bits(x.astype(np.float32)) for x in (q, k, v))
    g, kap, mg = _run(q, k, v, fmt, False)
    ref, rk, bd, inf = _oracle_heads(q, k, v, [fmt], False)
    assert np.all(rk[0, [5, 77, 200]] > 64)
    _check(g, kap, mg, ref, rk, bd, inf)
    # the whole tensor far above the guess: every row takes the re-based path
    g, kap, mg = _run(q, k, v, fmt, False, guess_bias=-100.0)
    ref, rk, bd, inf = _oracle_heads(q, k, v, [fmt], False, bias=-100.0)
    assert np.all(rk > 64)
    _check(g, kap, mg, ref, rk, bd, inf)
    # beyond the offsets the first pass records (321 binades): the fallback
    # pass measures them again from the scores
    g, kap, mg = _run(q, k, v, fmt, False, guess_bias=-400.0)
    ref, rk, bd, inf = _oracle_heads(q, k, v, [fmt], False, bias=-400.0)
    assert np.all(rk > 321)
    _check(g, kap, mg, ref, rk, bd, inf)


def test_tiny_workload_parity_and_error_criterion():
    w = W.WORKLOADS["tiny"]
    announce("fsa tiny workload")
    q, k, v = W.generate(w)
    g, kap, mg = _run(q, k, v, "e4m3")
    _check(g, kap, mg, *_oracle_heads(q, k, v, list(w.head_fmts)))
    ex, pl = [], []
    for h in range(w.H):
        qh, kh, vh = (W.bf16_bits_to_f64(x[0, h]) for x in (q, k, v))
        ex.append(O.exact_attention(qh, kh, vh))
        pl.append(O.plain_mx_attention(qh, kh, vh, "e4m3"))
    ex, pl = np.stack(ex), np.stack(pl)
    assert rel_l2(g[0], ex) <= 1.1 * rel_l2(pl, ex)


def test_deterministic():
    announce("fsa determinism")
    q, k, v = (W.random_bf16((1, 4, 1000, 128), seed, 1.0) for seed in (12, 13, 14))
    a, _, _ = _run(q, k, v, "e2m1")
    b, _, _ = _run(q, k, v, "e2m1")
    assert np.array_equal(a, b)


@pytest.mark.parametrize("fmt", FMTS)
def test_causal_many_tiles_sampled(fmt):
    """Causal rows across 16 key tiles: masked tiles at every ring phase and
    rows whose clean-tile count ranges over the whole sweep."""
    announce("fsa causal many tiles", fmt)
    S, D = 2000, 128
    q, k, v = (W.random_bf16((1, 2, S, D), seed, 1.2) for seed in (21, 22, 23))
    g, kap, mg = _run(q, k, v, fmt, True)
    rows = np.array([0, 1, 31, 127, 128, 129, 255, 256, 511, 640, 1023, 1024, 1151, 1500, 1919, 1999])
    for h in range(2):
        qh, kh, vh = (W.bf16_bits_to_f64(x[0, h]) for x in (q, k, v))
        ref, info = O.fused_attention(qh, kh, vh, fmt, True, rows=rows, return_info=True)
        ke = kappa_eps(info, fmt)
        border = kappa_rows(kappa_borderline(info["scores"], info["m_tilde"], rows, S, True,
                                             FORMATS[fmt].mbits, ke, low=kappa_low(fmt, "block")),
                            kappa_free(info, fmt, "block", ke), ke)
        skip = undecided(border, kap[0, h, rows], info["kappa"])
        assert excess_rel_l2(g[0, h, rows], ref, info, fmt, eps_rows(mg[0, h, rows], info, fmt),
                             skip=skip)[0] <= TOL
        check_kappa(kap[0, h, rows], info["kappa"], border)


@pytest.mark.parametrize("fmt", FMTS)
def test_rows_far_above_the_guess_causal(fmt):
    """The fallback pass with causal masking (planted rows past the window)."""
    announce("fsa far fallback causal", fmt)
    S, D = 400, 128
    q, k, v = (W.bf16_bits_to_f64(W.random_bf16((1, 1, S, D), seed, 1.0)) for seed in (31, 32, 33))
    c = O.attention.score_scale(D)
    for i, j in ((150, 140), (300, 290), (399, 131)):
        q[0, 0, i] = k[0, 0, j] * (300.0 / (c * float(k[0, 0, j] @ k[0, 0, j])))
    q, k, v = (W.f32_to_bf16_bits(x.astype(np.float32)) for x in (q, k, v))
    g, kap, mg = _run(q, k, v, fmt, True)
    ref, rk, bd, inf = _oracle_heads(q, k, v, [fmt], True)
    assert np.all(rk[0, [150, 300, 399]] > 64)
    _check(g, kap, mg, ref, rk, bd, inf)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("causal", [False, True])
def test_clustered_keys_under_the_capped_guess(fmt, causal):
    """Keys in two opposite clusters: the window's mean + z * std lies 200 to
    420 binades above each row's top score; the cap holds the guess at 64
    binades above the window max, so no row falls back.  Raised by a bias of
    150 binades, the same rows lie about 214 binades below their guess,
    beyond the reach of the scores' fp32 bit patterns (189 binades): the
    fallback pass measures their offsets from the scores and re-bases them
    downwards."""
    announce("fsa clustered keys", fmt, causal)
    q, k, v = W.two_valued_keys(1, 2, 600, 128, seed=41)
    g, kap, mg = _run(q, k, v, fmt, causal)
    ref, rk, bd, inf = _oracle_heads(q, k, v, [fmt] * 2, causal)
    assert np.all(rk == 0) and np.all(kap == 0)
    _check(g, kap, mg, ref, rk, bd, inf)
    g, kap, mg = _run(q, k, v, fmt, causal, guess_bias=150.0)
    ref, rk, bd, inf = _oracle_heads(q, k, v, [fmt] * 2, causal, bias=150.0)
    assert np.mean(rk < -189) > 0.9 and np.all(np.isfinite(g))
    _check(g, kap, mg, ref, rk, bd, inf)


@pytest.mark.parametrize("fmt", FMTS)
def test_largest_accepted_biases(fmt):
    """Guesses 1024 binades below and above every row (the bounds the
    library accepts): the first pass and the measure of each row's offset sum
    the scores around a reference 2^23 * 1213 from them, and every row still
    matches the oracle, re-based upwards or downwards by about 1024."""
    announce("fsa largest biases", fmt)
    q, k, v = (W.random_bf16((1, 1, 300, 128), seed, 1.0) for seed in (61, 62, 63))
    for bias in (-1024.0, 1024.0):
        g, kap, mg = _run(q, k, v, fmt, True, guess_bias=bias)
        ref, rk, bd, inf = _oracle_heads(q, k, v, [fmt], True, bias=bias)
        assert np.all(np.abs(rk + bias) < 100) and np.all(np.isfinite(g))
        _check(g, kap, mg, ref, rk, bd, inf)


def test_hybrid_heads_two_batches():
    """Per-head formats in one call with B = 2: each run of equal formats is
    quantised and launched per batch entry."""
    announce("fsa hybrid B=2")
    S, D = 300, 128
    fmts = ["e2m3", "e2m3", "e2m1", "e4m3"]
    q, k, v = (W.random_bf16((2, 4, S, D), seed, 1.1) for seed in (41, 42, 43))
    g, kap, mg = _run(q, k, v, "e2m3", False, head_fmt=fmts)
    _check(g, kap, mg, *_oracle_heads(q, k, v, fmts, False))


@pytest.mark.parametrize("fmts", [["e2m3", "e2m1", "e2m1", "e2m3", "e2m1", "e2m3"],
                                  ["e2m3", "e4m3", "e2m1", "e4m3", "e2m1", "e2m3"]],
                         ids=["fp6-fp4", "all-three"])
def test_hybrid_one_launch_strided(fmts):
    """Interleaved per-head formats in one launch, B = 2, over strided views:
    q, k and v stored [B, S, H, D] and read through [B, H, S, D] views, the
    output written into such a view too.  Every head must equal both the
    oracle and the same head computed alone in its format, contiguously
    (bit for bit: the same kernel body)."""
    import torch
    import softmax_mx_quantize_amd as fsa
    announce("fsa hybrid one launch strided", fmts)
    B, H, S, D = 2, len(fmts), 300, 128
    q, k, v = (W.random_bf16((B, H, S, D), seed, 1.2) for seed in (71, 72, 73))
    bshd = lambda x: to_dev(np.ascontiguousarray(x.transpose(0, 2, 1, 3))).transpose(1, 2)
    dq, dk, dv = bshd(q), bshd(k), bshd(v)
    assert not dq.is_contiguous()
    out = torch.empty((B, S, H, D), dtype=torch.bfloat16, device="cuda").transpose(1, 2)
    o, kap, mg = fsa.attention_fwd(dq, dk, dv, fmts[0], False, head_fmt=fmts, out=out, return_rows=True)
    torch.cuda.synchronize()
    g = from_dev_bf16(o.contiguous())
    _check(g, kap.cpu().numpy(), mg.cpu().numpy(), *_oracle_heads(q, k, v, fmts, False))
    for f in sorted(set(fmts)):
        alone = from_dev_bf16(fsa.attention_fwd(to_dev(q), to_dev(k), to_dev(v), f, False))
        heads = [h for h in range(H) if fmts[h] == f]
        assert np.array_equal(g[:, heads], alone[:, heads]), f


def test_workspace_grows_and_is_released():
    """Growing the workspace (stream-ordered) and releasing it leave results
    unchanged: a small call, a larger one, a release, the small one again."""
    import torch
    import softmax_mx_quantize_amd as fsa
    announce("fsa workspace growth")
    small = [W.random_bf16((1, 2, 200, 128), seed, 1.0) for seed in (101, 102, 103)]
    large = [W.random_bf16((1, 8, 3000, 128), seed, 1.0) for seed in (104, 105, 106)]
    a = fsa.attention_fwd(*(to_dev(x) for x in small), "e2m3")
    b = fsa.attention_fwd(*(to_dev(x) for x in large), "e2m3")
    torch.cuda.synchronize()
    fsa.release_workspace()
    c = fsa.attention_fwd(*(to_dev(x) for x in small), "e2m3")
    d = fsa.attention_fwd(*(to_dev(x) for x in large), "e2m3")
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), c.view(torch.int16))
    assert torch.equal(b.view(torch.int16), d.view(torch.int16))



def test_side_stream_calls_match_default_stream():
    """Calls on a stream other than the default one, with the workspace
    growing twice there (each old buffer freed on the stream that used it),
    give the default stream's results bit for bit; a later call back on the
    default stream does too."""
    import torch
    import softmax_mx_quantize_amd as fsa
    announce("fsa side stream")
    small = [to_dev(W.random_bf16((1, 2, 200, 128), seed, 1.0)) for seed in (111, 112, 113)]
    large = [to_dev(W.random_bf16((1, 8, 3000, 128), seed, 1.0)) for seed in (114, 115, 116)]
    ref_small = fsa.attention_fwd(*small, "e4m3")
    ref_large = fsa.attention_fwd(*large, "e4m3")
    torch.cuda.synchronize()
    fsa.release_workspace()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        a = fsa.attention_fwd(*small, "e4m3")
        b = fsa.attention_fwd(*large, "e4m3")
        c = fsa.attention_fwd(*small, "e4m3")
    side.synchronize()
    torch.cuda.current_stream().wait_stream(side)
    d = fsa.attention_fwd(*large, "e4m3")
    torch.cuda.synchronize()
    for got, want in ((a, ref_small), (b, ref_large), (c, ref_small), (d, ref_large)):
        assert torch.equal(got.view(torch.int16), want.view(torch.int16))


def test_host_threads_sharing_one_stream():
    """Calls from four host threads on one stream, sizes mixed so that the
    workspace grows meanwhile: every result equals the same call made alone
    (each call's kernels stay together on the stream)."""
    import threading
    import torch
    import softmax_mx_quantize_amd as fsa
    announce("fsa host threads")
    shapes = [(1, 2, 300, 128), (1, 6, 2500, 128), (2, 3, 700, 64), (1, 4, 4000, 128)]
    fmts = ["e4m3", "e2m1", "e2m3", "e4m3"]
    ins = [[to_dev(W.random_bf16(sh, 130 + 3 * t + j, 1.0)) for j in range(3)] for t, sh in enumerate(shapes)]
    refs = []
    for t in range(4):
        refs.append(fsa.attention_fwd(*ins[t], fmts[t]))
        torch.cuda.synchronize()
    fsa.release_workspace()
    outs = [[None] * 6 for _ in range(4)]
    errs = []

    def work(t):
        try:
            for r in range(6):
                outs[t][r] = fsa.attention_fwd(*ins[t], fmts[t])
        except Exception as e:                     # reported below
            errs.append(e)

    threads = [threading.Thread(target=work, args=(t,)) for t in range(4)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errs, errs
    for t in range(4):
        for r in range(6):
            assert torch.equal(outs[t][r].view(torch.int16), refs[t].view(torch.int16)), (t, r)


@pytest.mark.parametrize("case", ["q_zero", "k_zero", "v_const"])
def test_degenerate_inputs(case):
    """All-zero queries or keys (every score 0: uniform weights, the output
    is the mean of V^ over the visible keys) and a constant V (the output is
    that constant once quantised: -3.25 in E4M3 and E2M3, -3 in E2M1):
    against the oracle in every format, causal or not."""
    announce("fsa degenerate", case)
    S, D = 333, 128
    for fmt in FMTS:
        for causal in (False, True):
            q, k, v = (W.random_bf16((1, 2, S, D), seed, 1.3) for seed in (131, 132, 133))
            if case == "q_zero":
                q[:] = 0
            elif case == "k_zero":
                k[:] = 0
            else:
                v[:] = W.f32_to_bf16_bits(np.full(v.shape, -3.25, np.float32))
            g, kap, mg = _run(q, k, v, fmt, causal)
            ref, kaps, border, infos = _oracle_heads(q, k, v, [fmt] * 2, causal)
            _check(g, kap, mg, ref, kaps, border, infos)
            if case == "v_const":
                c = ref.ravel()[0]
                assert c == (-3.0 if fmt == "e2m1" else -3.25)
                assert np.all(ref == c) and np.all(g == c)

def test_skip_fallback_pass_hook():
    """Without the fallback pass, rows beyond the in-sweep shifts keep the
    first pass's offsets (65 binades or more); every other row is unchanged."""
    announce("fsa skip fallback pass")
    S, D = 300, 128
    q, k, v = (W.bf16_bits_to_f64(W.random_bf16((1, 1, S, D), seed, 1.0)) for seed in (12, 13, 14))
    c = O.attention.score_scale(D)
    far = [5, 77, 200]
    for i, j in zip(far, (140, 290, 131)):
        q[0, 0, i] = k[0, 0, j] * (300.0 / (c * float(k[0, 0, j] @ k[0, 0, j])))
    q, k, v = (W.f32_to_bf16_bits(x.astype(np.float32)) for x in (q, k, v))
    full, kf, _ = _run(q, k, v, "e2m1")
    part, kp, _ = _run(q, k, v, "e2m1", skip_fallback_pass=True)
    near = np.setdiff1d(np.arange(S), far)
    assert np.all(kp[0, 0, far] >= 65) and np.all(kf[0, 0, far] > 64)
    assert np.array_equal(part[0, 0, near], full[0, 0, near])
    assert np.array_equal(kp[0, 0, near], kf[0, 0, near])


@pytest.mark.parametrize("fmt,causal", [("e2m1", False), ("e4m3", True)])
def test_long_head_sampled_rows(fmt, causal):
    """One head of 2^21 + 37 keys (ragged last tile; key offsets and buffer
    ranges far past the workloads'): rows at both ends, at tile and block
    boundaries and in the middle, against the oracle over all keys."""
    import torch
    import softmax_mx_quantize_amd as fsa
    S, D = 2 ** 21 + 37, 128
    announce("fsa long head", fmt, causal, S)
    q, k, v = (W.random_bf16((1, 1, S, D), seed, 1.0) for seed in (61, 62, 63))
    rows = np.array([0, 1, 127, 128, 4097, S // 2 + 3, S - 130, S - 129, S - 38, S - 1])
    out, kap, mg = fsa.attention_fwd(to_dev(q), to_dev(k), to_dev(v), fmt, causal, return_rows=True)
    torch.cuda.synchronize()
    idx = torch.from_numpy(rows).cuda()
    g = from_dev_bf16(out[:, :, idx])
    kr = kap[:, :, idx].cpu().numpy()
    mr = mg[:, :, idx].cpu().numpy()
    del out, kap, mg
    ref, kaps, border, infos = _oracle_heads(q, k, v, [fmt], causal, rows=rows)
    info, f = infos[0]
    check_frozen_max(mr[0, 0], info, f)
    ex, _ = excess_rel_l2(g[0, 0], ref[0], info, f, eps_rows(mr[0, 0], info, f),
                          skip=undecided(border[0], kr[0, 0], kaps[0]))
    print("rel L2 %.2e, beyond near-tie codes %.2e" % (rel_l2(g[0, 0], ref[0]), ex))
    assert ex <= TOL, ex
    check_kappa(kr.ravel(), kaps.ravel(), border.ravel())


def test_many_heads_split_into_pieces():
    """300 heads (more than one launch's head table of 256, so the call runs
    in two pieces), cycling through the three formats, with per-row outputs:
    every row of every head against the oracle."""
    H, S, D = 300, 150, 64
    announce("fsa many heads", H)
    q, k, v = (W.random_bf16((1, H, S, D), seed, 1.2) for seed in (64, 65, 66))
    fmts = [FMTS[h % 3] for h in range(H)]
    g, kap, mg = _run(q, k, v, fmts[0], False, head_fmt=fmts)
    _check(g, kap, mg, *_oracle_heads(q, k, v, fmts, False))
