"""Shared plumbing for the GPU tests: host bf16 bits <-> device tensors."""

import sys

import numpy as np

import workloads as W


def announce(*what):
    print("[gpu case]", *what, flush=True)
    sys.stdout.flush()


def to_dev(bits: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def from_dev_bf16(t) -> np.ndarray:
    import torch
    bits = t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
    return W.bf16_bits_to_f64(bits)


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm((a - b).ravel()) / np.linalg.norm(b.ravel()))


_TENSOR_CACHE = {}


def workload_tensors(w):
    """bf16 bits of a workload's q, k, v, kept for the rest of the session:
    workloads that share a recipe (the Video-DiT formats) share one copy.
    At most two recipes are kept."""
    key = (w.B, w.H, w.S, w.D, w.seed, w.gain_range, w.outlier_frac, w.outlier_sigma,
           w.heavy_frac, w.heavy_nu)
    if key not in _TENSOR_CACHE:
        while len(_TENSOR_CACHE) >= 2:
            _TENSOR_CACHE.pop(next(iter(_TENSOR_CACHE)))
        _TENSOR_CACHE[key] = W.generate(w, workers=16)
    return _TENSOR_CACHE[key]


def kappa_borderline(scores, m_tilde, rows, S, causal, mbits, eps=2e-3, exact=False):
    """Rows whose fallback offset kappa may legitimately differ by one between
    the GPU and the oracle: kappa steps where the row's largest visible
    guess-relative score t_max crosses j - 2^-(M+1) (j >= 1), and the kernel
    carries t with fp32 placement, its own frozen max and fp32 sums, so rows
    within ``eps`` binades of such a step are borderline."""
    j = np.arange(S)[None, :]
    vis = (j <= np.asarray(rows)[:, None]) if causal else np.ones((len(rows), S), bool)
    t = np.where(vis, scores - np.asarray(m_tilde)[:, None], -np.inf).max(axis=1)
    if exact:
        # the exact value 2^t rounds up a binade at frac(t) = log2(2 - 2^-(M+1))
        step = 1.0 - np.log2(2.0 - 2.0 ** -(mbits + 1))
    else:
        step = 2.0 ** -(mbits + 1)
    jn = np.maximum(1.0, np.rint(t + step))
    return np.abs(t - (jn - step)) < eps


def check_kappa(gpu_kap, ref_kap, borderline):
    """Exact agreement outside the borderline rows, within one inside them."""
    gpu_kap = np.asarray(gpu_kap, np.int64)
    ref_kap = np.asarray(ref_kap, np.int64)
    bad = (gpu_kap != ref_kap) & ~(borderline & (np.abs(gpu_kap - ref_kap) <= 1))
    assert not bad.any(), ("kappa mismatch", np.flatnonzero(bad)[:10], gpu_kap[bad][:10], ref_kap[bad][:10])
    return int(borderline.sum())


def row_rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.linalg.norm(a - b, axis=-1) / np.linalg.norm(b, axis=-1)
