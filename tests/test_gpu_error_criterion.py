"""Acceptance criterion 3 at the full workload sizes: against float64 exact
attention, the fused-softmax output's error stays within 1.1x that of plain
exp-then-quantize MX attention on the same operands (Fused-Softmax for
efficient quantized attention, summary: the added error stays below the
quantisation floor).  Both MX paths multiply the same pre-scaled q'^, k^ and
v^, so the comparison isolates the approximated exponential and the frozen
max.

Every head of every workload is evaluated on its own sample of query rows
(relL2 = ||a - b|| / ||b|| over the sample); the GPU output comes from one
call over the whole tensor.  Asserted:

* per workload, the ratio pooled over all heads' rows is at most 1.1;
* per head, the ratio is at most 1.1 unless its sampling spread explains the
  excess: the per-row errors are heavy-tailed (a few rows whose weight sits
  on a handful of keys dominate a few hundred rows), so the head must not be
  above 1.1 by more than three bootstrap standard deviations over its rows.

Every per-head ratio and its spread is printed.
"""

import concurrent.futures
import os

import numpy as np
import pytest

import workloads as W
import oracle as O
from gpu_helpers import announce, to_dev, from_dev_bf16, workload_tensors

pytestmark = pytest.mark.gpu

CASES = [("video_dit_e4m3", 512), ("video_dit_e2m3", 512), ("video_dit_e2m1", 512),
         ("outliers_e2m1", 384), ("hybrid_long", 256)]
BAR = 1.1


def _threads():
    try:
        n = len(os.sched_getaffinity(0))
    except Exception:
        n = os.cpu_count() or 4
    return max(1, min(16, n))


def _head_errors(w, h, qkv, rows, g_rows):
    """Per-row squared errors of the GPU output and of the plain MX path
    against exact attention for one head (oracle on the host)."""
    qh, kh, vh = (W.bf16_bits_to_f64(x[0, h]) for x in qkv)
    ex = O.exact_attention(qh, kh, vh, w.causal, rows=rows)
    pl = O.plain_mx_attention(qh, kh, vh, w.head_fmts[h], w.causal, rows=rows)
    ef = np.sum((g_rows - ex) ** 2, axis=1)
    ep = np.sum((pl - ex) ** 2, axis=1)
    return ef, ep


@pytest.mark.parametrize("name,n_rows", CASES, ids=[c[0] for c in CASES])
def test_fused_error_within_1p1_of_plain_mx_per_head(name, n_rows):
    import torch
    import softmax_mx_quantize_amd as fsa
    w = W.WORKLOADS[name]
    announce("error criterion", name, "rows per head", n_rows)
    q, k, v = workload_tensors(w)
    hf = list(w.head_fmts)
    kw = {} if len(set(hf)) == 1 else {"head_fmt": hf}
    out = fsa.attention_fwd(to_dev(q), to_dev(k), to_dev(v), hf[0], w.causal, **kw)
    torch.cuda.synchronize()
    g = from_dev_bf16(out)
    del out
    samples = {h: np.sort(np.random.default_rng([77, h]).choice(w.S, n_rows, replace=False))
               for h in range(w.H)}
    res = {}
    with concurrent.futures.ThreadPoolExecutor(_threads()) as ex:
        futs = {ex.submit(_head_errors, w, h, (q, k, v), samples[h], g[0, h, samples[h]]): h
                for h in range(w.H)}
        for f in concurrent.futures.as_completed(futs):
            res[futs[f]] = f.result()
            print("  oracle done for head %d (%d of %d)" % (futs[f], len(res), w.H), flush=True)
    rng = np.random.default_rng(5)
    worst, EF, EP = [], 0.0, 0.0
    for h in range(w.H):
        ef, ep = res[h]
        EF += ef.sum()
        EP += ep.sum()
        ratio = float(np.sqrt(ef.sum() / ep.sum()))
        idx = rng.integers(0, ef.size, size=(400, ef.size))
        boot = np.sqrt(ef[idx].sum(axis=1) / ep[idx].sum(axis=1))
        sd = float(boot.std())
        print("%s head %2d (%s): ratio %.3f  bootstrap sd %.3f" % (name, h, hf[h], ratio, sd))
        if ratio > BAR:
            worst.append((h, ratio, sd))
    pooled = float(np.sqrt(EF / EP))
    print("%s pooled ratio %.3f over %d heads x %d rows; heads above %.1f: %s"
          % (name, pooled, w.H, n_rows, BAR, worst))
    assert pooled <= BAR, pooled
    for h, ratio, sd in worst:
        assert ratio <= BAR + 3.0 * sd, (h, ratio, sd)
