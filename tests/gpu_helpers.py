"""Shared plumbing for the GPU tests: host bf16 bits <-> device tensors."""

import sys

import numpy as np

import workloads as W
from parity import frozen_max_tol


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


def kappa_borderline(scores, m_tilde, rows, S, causal, mbits, eps=2e-3, exact=False, low=None):
    """Rows whose fallback offset kappa may legitimately differ by one between
    the GPU and the oracle: kappa steps where the row's largest visible
    guess-relative score t_max crosses j - 2^-(M+1) (j >= 1, and below
    ``low``, the low-side threshold of kappa_low, every j), and the kernel
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
    jr = np.rint(t + step)
    jn = np.maximum(1.0, jr) if low is None else np.where(t < low, jr, np.maximum(1.0, jr))
    return np.abs(t - (jn - step)) < eps


def kappa_low(pfmt, mode):
    """The guess-relative t_max below which a row is re-based downwards: its
    top block then needs a shift beyond 127 - pl binades (block modes), or
    its largest value rounds to zero (one scale per row)."""
    from oracle import FORMATS
    from oracle.attention import placement_exponent
    f = FORMATS[pfmt]
    M = f.mbits
    pl = placement_exponent(f)
    if mode == "row":
        return -f.bias - M - pl                # Mitchell value 2^thr: half the least subnormal
    step = 1.0 - np.log2(2.0 - 2.0 ** -(M + 1)) if mode == "exp" else 2.0 ** -(M + 1)
    return -(127 - pl) - step


def check_frozen_max(gpu_m_tilde, info, fmt=None):
    """The kernel's frozen max against the oracle's, within frozen_max_tol
    (tests/parity.py)."""
    dm = np.abs(np.asarray(gpu_m_tilde, np.float64) - info["m_tilde"])
    tol = frozen_max_tol(info, fmt)
    assert np.all(dm <= tol), (float(dm.max()), int(np.argmax(dm - tol)))


def kappa_free(info, pfmt, mode, eps):
    """Rows within ``eps`` binades (per row) of the low-side threshold
    (kappa_low): on its two sides kappa is 0 or about -(127 - pl) (-17 with
    one scale per row), so such rows are left free."""
    t = np.where(info["visible"], info["scores"] - info["m_tilde"][:, None], -np.inf).max(axis=1)
    return np.abs(t - kappa_low(pfmt, mode)) < eps


def kappa_rows(border, free, eps=None):
    """Per-row codes for check_kappa: bit 0 borderline (kappa may differ by
    one, or by ceil(eps) where the row's margin ``eps`` spans more than a
    binade: scores thousands of binades large carry FP8 errors of whole
    binades), bit 1 free (kappa unchecked), the extra slack from bit 2 on."""
    code = np.asarray(border).astype(np.int32) + 2 * np.asarray(free).astype(np.int32)
    if eps is not None:
        extra = np.maximum(0, np.ceil(np.asarray(eps, np.float64)) - 1).astype(np.int32)
        code = code + 4 * np.where(np.asarray(border), extra, 0)
    return code


def check_kappa(gpu_kap, ref_kap, borderline):
    """Exact agreement outside the borderline rows, within their slack
    (one, or more: kappa_rows) inside them; free rows are not checked."""
    gpu_kap = np.asarray(gpu_kap, np.int64)
    ref_kap = np.asarray(ref_kap, np.int64)
    code = np.asarray(borderline).astype(np.int64)
    slack = 1 + (code >> 2)
    d = np.abs(gpu_kap - ref_kap)
    bad = (d > 0) & ~(((code & 1) != 0) & (d <= slack)) & ((code & 2) == 0)
    assert not bad.any(), ("kappa mismatch", np.flatnonzero(bad)[:10], gpu_kap[bad][:10], ref_kap[bad][:10])
    return int(np.count_nonzero(code))


def row_rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.linalg.norm(a - b, axis=-1) / np.linalg.norm(b, axis=-1)
