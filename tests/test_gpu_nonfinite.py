"""Non-finite inputs through the fused attention, against the oracle.

A NaN or Inf element makes its MX block's scale NaN (byte 0xFF; OCP MX), so
a NaN in K makes every score against that key NaN, one in Q every score of
that query, one in V that output column.  The oracle follows IEEE
propagation through softmax, as exact attention does: a row is NaN wherever
it sees a NaN score (a causal row does not see later keys), and a V block's
NaN reaches its output column in every row.  The GPU must give the same NaN
pattern, and the finite part must match the oracle as elsewhere.
"""

import numpy as np
import pytest

import workloads as W
import oracle as O
from gpu_helpers import announce, to_dev, from_dev_bf16, rel_l2

pytestmark = pytest.mark.gpu

S, D = 300, 128
# (tensor, row, column, value): a key beyond the frozen max's window, one
# inside it, a query, a value, an infinite key
PLANTS = {
    "k_late": ("k", 200, 5, np.nan),
    "k_window": ("k", 50, 5, np.nan),
    "k_inf": ("k", 220, 9, np.inf),
    "q": ("q", 7, 3, np.nan),
    "v": ("v", 100, 40, np.nan),
}


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("where", list(PLANTS))
def test_nonfinite_inputs_propagate_like_the_oracle(where, causal, fmt):
    import torch
    import softmax_mx_quantize_amd as fsa
    announce("fsa non-finite", where, causal, fmt)
    t, r, c, val = PLANTS[where]
    x = {n: W.random_bf16((1, 1, S, D), seed, 1.0) for n, seed in (("q", 121), ("k", 122), ("v", 123))}
    x[t][0, 0, r, c] = W.f32_to_bf16_bits(np.array([val], np.float32))[0]
    out = fsa.attention_fwd(to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"]), fmt, causal)
    torch.cuda.synchronize()
    g = from_dev_bf16(out)[0, 0]
    qh, kh, vh = (W.bf16_bits_to_f64(x[n][0, 0]) for n in ("q", "k", "v"))
    with np.errstate(invalid="ignore", over="ignore", divide="ignore"):
        ref = O.fused_attention(qh, kh, vh, fmt, causal)
    nan_ref, nan_gpu = np.isnan(ref), np.isnan(g)
    assert nan_ref.any()
    assert np.array_equal(nan_gpu, nan_ref), (np.flatnonzero(nan_gpu.any(1)), np.flatnonzero(nan_ref.any(1)))
    # the finite part: whole rows untouched by the planted value
    fin = ~nan_ref.any(axis=1)
    if fin.any():
        err = rel_l2(g[fin], ref[fin])
        print("finite rows %d, rel L2 %.2e" % (fin.sum(), err))
        assert err <= 2e-3, err
