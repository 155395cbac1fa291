"""The allocation-free entry point (fsa_attention_fwd_noalloc, fixed device
scratch) against the allocating fsa_attention_fwd_ex, through the C ABI.

Both run the same kernels on the same inputs; grouping heads into scratch-
sized pieces changes no row's arithmetic, so outputs, fallback offsets and
frozen maxima must agree bit for bit (stronger than the 2e-3 parity bar).
Two calls in a row, the second smaller; the first spans several scratch
pieces (two per batch entry, two batch entries) and mixed formats, and one
case forces every row through the fallback pass, which reads its per-row
arrays back from the scratch.  A captured graph of one call replays
correctly on new inputs.
"""

import numpy as np
import pytest

import workloads as W
from gpu_helpers import announce, to_dev

pytestmark = pytest.mark.gpu


def _both(q, k, v, fmt, causal=False, **kw):
    import torch
    import softmax_mx_quantize_amd as fsa
    dq, dk, dv = to_dev(q), to_dev(k), to_dev(v)
    a = fsa.attention_fwd(dq, dk, dv, fmt, causal, **kw)
    b = fsa.attention_fwd(dq, dk, dv, fmt, causal, no_alloc=True, **kw)
    torch.cuda.synchronize()
    return a, b


def _same(a, b):
    import torch
    if isinstance(a, tuple):
        for x, y in zip(a, b):
            assert torch.equal(x, y)
    else:
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_noalloc_equals_allocating_call_twice():
    # first call: 8 heads of S = 50000 at FP8 need about 109 MB, so the 64 MiB
    # scratch takes them four at a time (two pieces per batch entry)
    B, H, S, D = 2, 8, 50000, 128
    announce("no-alloc first call", B, H, S, D)
    q, k, v = (W.random_bf16((B, H, S, D), seed, 1.1) for seed in (61, 62, 63))
    a, b = _both(q, k, v, "e4m3")
    _same(a, b)
    a, b = _both(q, k, v, "e4m3", return_rows=True)
    _same(a, b)
    hf = ["e4m3"] * 5 + ["e2m1"] * 2 + ["e2m3"]
    a, b = _both(q, k, v, "e4m3", head_fmt=hf)
    _same(a, b)
    del q, k, v
    # second call, smaller: causal, and every row through the fallback pass
    B, H, S = 1, 3, 1000
    announce("no-alloc second call", B, H, S, D)
    q, k, v = (W.random_bf16((B, H, S, D), seed, 1.0) for seed in (64, 65, 66))
    a, b = _both(q, k, v, "e2m3", True)
    _same(a, b)
    a, b = _both(q, k, v, "e2m1", False, guess_bias=-100.0)
    _same(a, b)
    a, b = _both(q, k, v, "e2m1", False, guess_bias=-100.0, return_rows=True)
    _same(a, b)
    assert bool((a[1] > 64).all())


def test_noalloc_rejects_a_head_beyond_the_scratch():
    import torch
    import softmax_mx_quantize_amd as fsa
    S, D = 260000, 128                      # one FP8 head needs ~70 MB
    announce("no-alloc too large", S)
    q = torch.zeros((1, 1, S, D), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fsa.FsaError) as e:
        fsa.attention_fwd(q, q.clone(), q.clone(), "e4m3", no_alloc=True)
    assert e.value.status == -5
    # the allocating call takes it
    out = fsa.attention_fwd(q, q.clone(), q.clone(), "e4m3")
    torch.cuda.synchronize()
    assert out.shape == q.shape


@pytest.mark.parametrize("fmt,causal", [("e4m3", False), ("e2m1", True)])
def test_noalloc_call_replays_in_a_graph(fmt, causal):
    """One allocation-free call captured in a graph, replayed on three sets
    of inputs copied into its static tensors, with eager calls and
    synchronisations between the replays: every replay equals an eager
    allocation-free call on the same inputs, bit for bit (the path records
    no memset and no allocation)."""
    import torch
    import softmax_mx_quantize_amd as fsa
    announce("no-alloc graph", fmt, causal)
    B, H, S, D = 1, 3, 700, 128
    sets = [[to_dev(W.random_bf16((B, H, S, D), 3000 + 3 * r + j, 1.0 + 0.3 * r)) for j in range(3)]
            for r in range(3)]
    sq, sk, sv = (torch.empty_like(x) for x in sets[0])
    sout = torch.empty_like(sq)
    for x, y in zip((sq, sk, sv), sets[0]):
        x.copy_(y)
    # the first call on the device looks up the scratch's address: eager, before capture
    fsa.attention_fwd(sq, sk, sv, fmt, causal, no_alloc=True, out=sout)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            fsa.attention_fwd(sq, sk, sv, fmt, causal, no_alloc=True, out=sout)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for r in range(3):
        for x, y in zip((sq, sk, sv), sets[r]):
            x.copy_(y)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = sout.clone()
        want = fsa.attention_fwd(*sets[r], fmt, causal, no_alloc=True)
        other = fsa.attention_fwd(*sets[(r + 1) % 3], fmt, causal)      # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), r
        assert other.shape == got.shape
