"""Acceptance criterion 3 at the full workload sizes: against float64 exact
attention, the fused-softmax output's error stays within 1.1x that of plain
exp-then-quantize MX attention on the same operands (Fused-Softmax for
efficient quantized attention, summary: the added error stays below the
quantisation floor).

Evaluated per workload over sampled query rows of 14 heads (6 for the hybrid
schedule), pooled over those rows: relL2 = ||a - b|| / ||b|| over all sampled
elements.  Per-head ratios are printed; with a few dozen rows per head they
scatter about 1 (0.44-1.56 measured), so the bar is the pooled one.
"""

import numpy as np
import pytest

import workloads as W
import oracle as O
from gpu_helpers import announce, to_dev, from_dev_bf16, rel_l2

pytestmark = pytest.mark.gpu

CASES = [("video_dit_e4m3", tuple(range(0, 40, 3)), 24),
         ("video_dit_e2m3", tuple(range(0, 40, 3)), 24),
         ("video_dit_e2m1", tuple(range(0, 40, 3)), 24),
         ("outliers_e2m1", (0, 13, 27), 16),
         ("hybrid_long", (0, 10, 19, 20, 30, 39), 8)]


@pytest.mark.parametrize("name,heads,n_rows", CASES, ids=[c[0] for c in CASES])
def test_fused_error_within_1p1_of_plain_mx(name, heads, n_rows):
    import torch
    import softmax_mx_quantize_amd as fsa
    w = W.WORKLOADS[name]
    announce("error criterion", name)
    q, k, v = W.generate(w)
    hf = list(w.head_fmts)
    kw = {} if len(set(hf)) == 1 else {"head_fmt": hf}
    out = fsa.attention_fwd(to_dev(q), to_dev(k), to_dev(v), hf[0], w.causal, **kw)
    torch.cuda.synchronize()
    g = from_dev_bf16(out)
    rng = np.random.default_rng(99)
    rows = np.sort(rng.choice(w.S, size=n_rows, replace=False))
    G, E, P = [], [], []
    for h in heads:
        qh, kh, vh = (W.bf16_bits_to_f64(x[0, h]) for x in (q, k, v))
        ex = O.exact_attention(qh, kh, vh, w.causal, rows=rows)
        pl = O.plain_mx_attention(qh, kh, vh, hf[h], w.causal, rows=rows)
        gh = g[0, h, rows]
        print("%s head %d (%s): fused %.3e, plain %.3e, ratio %.3f"
              % (name, h, hf[h], rel_l2(gh, ex), rel_l2(pl, ex), rel_l2(gh, ex) / rel_l2(pl, ex)))
        G.append(gh)
        E.append(ex)
        P.append(pl)
    G, E, P = np.stack(G), np.stack(E), np.stack(P)
    ratio = rel_l2(G, E) / rel_l2(P, E)
    print("%s pooled ratio %.3f" % (name, ratio))
    assert ratio <= 1.1, ratio
