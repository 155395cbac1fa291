"""Seeded synthetic inputs for fused-softmax attention.

This module only draws random numbers and rounds them to bfloat16. It holds
none of the attention or quantisation arithmetic, so that the CPU oracle and
the GPU path can both read the very same input bytes without sharing any
method code.

Every tensor is bf16 ``[B, H, S, D]``, row-major, returned as ``uint16`` bit
patterns.  Each (tensor, batch, head) slice is drawn from its own
``numpy.random.default_rng`` stream keyed by ``(seed, tensor, b, h)``, so a
single head can be regenerated without drawing the others.

The workloads mirror the shapes the fused-softmax pages talk about (video
diffusion attention with 40 heads of width 128; Fused-Softmax for efficient
quantized attention, summary) with synthetic values: no model weights or
activations are available, so Gaussian inputs stand in for them.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

# Element formats by name; the integer values match the C ABI's enum.
FMT_IDS = {"e4m3": 0, "e2m3": 1, "e2m1": 2}

_T_Q, _T_K, _T_V, _T_GAIN, _T_OUTLIER, _T_HEAVY = 0, 1, 2, 3, 4, 5


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    S: int
    D: int
    causal: bool
    seed: int
    head_fmts: Tuple[str, ...]      # element format per head
    gain_range: Optional[Tuple[float, float]] = None   # per-head gain on q and k
    outlier_frac: float = 0.0       # fraction of query rows given one +8 sigma score
    outlier_sigma: float = 8.0
    heavy_frac: float = 0.0         # fraction of key positions with Student-t rows
    heavy_nu: float = 4.0

    @property
    def flops(self) -> float:
        """Attention FLOPs: 2*S*S*D for Q K^T plus the same for P V, per head."""
        f = 4.0 * self.B * self.H * self.S * self.S * self.D
        return f / 2 if self.causal else f


def _uniform_fmt(fmt: str, H: int) -> Tuple[str, ...]:
    return tuple([fmt] * H)


WORKLOADS: Dict[str, Workload] = {
    # Small case that the oracle finishes in seconds.
    "tiny": Workload("tiny", 1, 2, 256, 64, False, 0, _uniform_fmt("e4m3", 2)),
    # Video-DiT-shaped attention, per-head gain so that the score std spans
    # about 0.25 .. 4 in softmax-scaled units.
    "video_dit_e4m3": Workload("video_dit_e4m3", 1, 40, 16384, 128, False, 1,
                               _uniform_fmt("e4m3", 40), gain_range=(0.5, 2.0)),
    # The same tensors with E2M3 elements (the BF16 kernel is timed on them too).
    "video_dit_e2m3": Workload("video_dit_e2m3", 1, 40, 16384, 128, False, 1,
                               _uniform_fmt("e2m3", 40), gain_range=(0.5, 2.0)),
    # The same tensors with E2M1 elements.
    "video_dit_e2m1": Workload("video_dit_e2m1", 1, 40, 16384, 128, False, 1,
                               _uniform_fmt("e2m1", 40), gain_range=(0.5, 2.0)),
    # The Video-DiT E4M3 tensors with causal masking (key j visible to query
    # i iff j <= i): the masked tiles and the causal tile skipping.
    "video_dit_e4m3_causal": Workload("video_dit_e4m3_causal", 1, 40, 16384, 128, True, 1,
                                      _uniform_fmt("e4m3", 40), gain_range=(0.5, 2.0)),
    # E2M1 with planted +8 sigma scores in 1 % of the query rows.
    "outliers_e2m1": Workload("outliers_e2m1", 1, 40, 32768, 128, False, 3,
                              _uniform_fmt("e2m1", 40), outlier_frac=0.01),
    # Long sequence, hybrid E2M3 / E2M1 heads, heavy-tailed keys.
    "hybrid_long": Workload("hybrid_long", 1, 40, 75600, 128, False, 4,
                            tuple(["e2m3"] * 20 + ["e2m1"] * 20), heavy_frac=0.05),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns uint16 bits."""
    b = np.array(x, dtype=np.float32, copy=True).view(np.uint32)
    t = np.right_shift(b, np.uint32(16))
    np.bitwise_and(t, np.uint32(1), out=t)
    np.add(t, np.uint32(0x7FFF), out=t)
    np.add(b, t, out=b)
    np.right_shift(b, np.uint32(16), out=b)
    return b.astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact float64 values of bfloat16 bit patterns."""
    u = bits.astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def _rng(seed: int, tensor: int, b: int, h: int) -> np.random.Generator:
    return np.random.default_rng([seed, tensor, b, h])


def head_gain(w: Workload, b: int, h: int) -> float:
    if w.gain_range is None:
        return 1.0
    lo, hi = w.gain_range
    return float(_rng(w.seed, _T_GAIN, b, h).uniform(lo, hi))


def generate_head(w: Workload, b: int, h: int,
                  S: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """bf16 bits of q, k, v for one (batch, head) slice, each ``[S, D]``.

    ``S`` may shrink the sequence (the first ``S`` rows of the same streams
    are not reproduced in general; shrinking draws a smaller problem with the
    same recipe).
    """
    S = w.S if S is None else S
    D = w.D
    g = np.float32(head_gain(w, b, h))
    q = _rng(w.seed, _T_Q, b, h).standard_normal((S, D), dtype=np.float32) * g
    k = _rng(w.seed, _T_K, b, h).standard_normal((S, D), dtype=np.float32) * g
    v = _rng(w.seed, _T_V, b, h).standard_normal((S, D), dtype=np.float32)
    if w.heavy_frac > 0.0:
        r = _rng(w.seed, _T_HEAVY, b, h)
        n = int(round(w.heavy_frac * S))
        pos = r.choice(S, size=n, replace=False)
        k[pos] = r.standard_t(w.heavy_nu, size=(n, D)).astype(np.float32)
    kb = f32_to_bf16_bits(k)
    if w.outlier_frac > 0.0:
        # Give each chosen row one key whose raw score is outlier_sigma * sqrt(D),
        # i.e. +8 standard deviations of a unit-variance score after the 1/sqrt(D)
        # softmax scale.  q_i is rotated toward k_j with its norm kept, so the
        # row's other scores keep their spread.  The key lies outside the first
        # 128 keys.
        r = _rng(w.seed, _T_OUTLIER, b, h)
        n = int(math.floor(w.outlier_frac * S))
        rows = r.choice(S, size=n, replace=False)
        keys = r.integers(min(128, S - 1), S, size=n)
        kf = bf16_bits_to_f64(kb)
        target = w.outlier_sigma * math.sqrt(D)
        for i, j in zip(rows, keys):
            kj = kf[j]
            u = kj / np.linalg.norm(kj)
            qi = q[i].astype(np.float64)
            c = target / np.linalg.norm(kj)               # wanted component along k_j
            perp = qi - (qi @ u) * u
            rest = max(qi @ qi - c * c, 0.0)
            qi = c * u + math.sqrt(rest) * perp / max(np.linalg.norm(perp), 1e-30)
            q[i] = qi.astype(np.float32)
    return f32_to_bf16_bits(q), kb, f32_to_bf16_bits(v)


def outlier_rows(w: Workload, b: int, h: int) -> np.ndarray:
    """Query rows that received a planted outlier score (empty if none)."""
    if w.outlier_frac <= 0.0:
        return np.zeros(0, dtype=np.int64)
    r = _rng(w.seed, _T_OUTLIER, b, h)
    n = int(math.floor(w.outlier_frac * w.S))
    return np.sort(r.choice(w.S, size=n, replace=False))


def generate(w: Workload, S: Optional[int] = None,
             workers: int = 8) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """bf16 bits of q, k, v, each ``[B, H, S, D]`` (all heads), as uint16.

    Heads are drawn in parallel threads; each head has its own streams, so
    the result does not depend on the number of workers.
    """
    import concurrent.futures
    S = w.S if S is None else S
    shape = (w.B, w.H, S, w.D)
    q = np.empty(shape, np.uint16)
    k = np.empty(shape, np.uint16)
    v = np.empty(shape, np.uint16)

    def one(bh):
        b, h = bh
        q[b, h], k[b, h], v[b, h] = generate_head(w, b, h, S)

    jobs = [(b, h) for b in range(w.B) for h in range(w.H)]
    with concurrent.futures.ThreadPoolExecutor(max_workers=max(1, workers)) as ex:
        list(ex.map(one, jobs))
    return q, k, v


def random_bf16(shape, seed: int, scale: float = 1.0) -> np.ndarray:
    """Plain N(0, scale^2) bf16 bits for unit tests of arbitrary shapes."""
    x = np.random.default_rng(seed).standard_normal(shape, dtype=np.float32) * np.float32(scale)
    return f32_to_bf16_bits(x)


def two_valued_keys(B: int, H: int, S: int, D: int, seed: int, a: float = 1.9,
                    gain=(1.0, 2.0), noise: float = 0.3, period: int = 2):
    """Q, K, V bf16 bits [B, H, S, D] whose keys take two opposite directions:
    k_j = +a for j a multiple of ``period``, -a otherwise, plus N(0, noise^2)
    per element, and q_i = r_i a with r_i uniform in ``gain``, plus the same
    noise.  Every row's scores split into a high and a low cluster, a light
    upper tail: a guess built from the window's mean and spread lands far
    above the row's top score (with period 2 by about 3.6 times the top)."""
    rng = np.random.default_rng(seed)
    sign = np.where(np.arange(S) % period == 0, 1.0, -1.0)[:, None]
    r = rng.uniform(gain[0], gain[1], size=(B, H, S, 1))
    q = r * a + noise * rng.standard_normal((B, H, S, D))
    k = sign * a + noise * rng.standard_normal((B, H, S, D))
    v = rng.standard_normal((B, H, S, D))
    return tuple(f32_to_bf16_bits(x.astype(np.float32)) for x in (q, k, v))
