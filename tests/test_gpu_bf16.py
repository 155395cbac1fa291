"""BF16 flash-attention baseline on the GPU against float64 exact attention."""

import numpy as np
import pytest

import workloads as W
import oracle as O
from gpu_helpers import announce, to_dev, from_dev_bf16, rel_l2

pytestmark = pytest.mark.gpu

# bf16 P and bf16 output each round to 8 significant bits (2^-9 relative);
# the output's relative L2 error stays well under 5e-3.
TOL = 5e-3


def _run(q, k, v, causal):
    import torch
    import softmax_mx_quantize_amd as fsa
    out = fsa.attention_bf16_ref(to_dev(q), to_dev(k), to_dev(v), causal)
    torch.cuda.synchronize()
    return from_dev_bf16(out)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("S", [1, 77, 300, 1030])
def test_bf16_matches_exact(D, causal, S):
    announce("bf16", D, causal, S)
    q, k, v = (W.random_bf16((1, 2, S, D), seed, 1.5) for seed in (21, 22, 23))
    g = _run(q, k, v, causal)
    for h in range(2):
        qh, kh, vh = (W.bf16_bits_to_f64(x[0, h]) for x in (q, k, v))
        ex = O.exact_attention(qh, kh, vh, causal)
        assert rel_l2(g[0, h], ex) <= TOL


def test_bf16_full_size_sampled():
    w = W.WORKLOADS["video_dit_e2m3"]
    announce("bf16 full size")
    q, k, v = W.generate(w)
    g = _run(q, k, v, False)
    rows = np.sort(np.random.default_rng(3).choice(w.S, 32, replace=False))
    for h in (0, 20, 39):
        qh, kh, vh = (W.bf16_bits_to_f64(x[0, h]) for x in (q, k, v))
        ex = O.exact_attention(qh, kh, vh, False, rows)
        assert rel_l2(g[0, h, rows], ex) <= TOL


@pytest.mark.parametrize("causal", [False, True])
def test_bf16_growing_scores(causal):
    """Scores that climb by about 100 binades along the keys (about 6 per
    64-key tile) move the kept row max past its 8-binade margin every tile
    or two, which exercises the rescale of the output and the row sum."""
    S, D = 1030, 128
    announce("bf16 growing scores", causal)
    rng = np.random.default_rng(31)
    u = rng.standard_normal(D)
    u /= np.linalg.norm(u)
    q = np.tile(20.0 * u, (S, 1)) + 0.1 * rng.standard_normal((S, D))
    ramp = 40.0 * np.arange(S) / S
    k = ramp[:, None] * u[None, :] + 0.1 * rng.standard_normal((S, D))
    v = rng.standard_normal((S, D))
    q, k, v = (W.f32_to_bf16_bits(x.astype(np.float32))[None, None] for x in (q, k, v))
    g = _run(q, k, v, causal)
    qh, kh, vh = (W.bf16_bits_to_f64(x[0, 0]) for x in (q, k, v))
    ex = O.exact_attention(qh, kh, vh, causal)
    assert np.all(np.isfinite(g))
    assert rel_l2(g[0, 0], ex) <= TOL
