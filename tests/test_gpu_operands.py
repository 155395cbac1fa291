"""Acceptance criterion 1 on the attention path: the MX codes and E8M0 scales
the fused kernels consume match the oracle bit for bit.

``fsa_debug_operands`` returns Q'^ as quantised by the attention kernel's
own prologue code (scale bytes raised by 23, the 2^23 the kernel folds into
Q's scale), and K^ / V^T exactly as they sit in the workspace, their scales
in the tile orders the products read.  The tile orders are mapped back here
from their description in include/fsa.h (written out independently of the
library's layout functions).
"""

import numpy as np
import pytest

import workloads as W
import oracle as O
from oracle.attention import prescale_q
from gpu_helpers import announce, to_dev

pytestmark = pytest.mark.gpu
BITS = {"e4m3": 8, "e2m3": 6, "e2m1": 4}


def key_tile_position(kk, blk, D, bits):
    """Byte of key row kk (0..127) and D block blk in one key tile."""
    u, r = kk // 64, kk % 64
    j, k4 = (r // 4) % 4, r % 4
    if bits == 8:
        x, beta = (r // 16) % 2, r // 32
    else:
        x, beta = r // 32, (r // 16) % 2
    rho = 8 * j + 4 * x + k4
    return (32 * (blk % 2) + rho) * (D // 16) + u * (D // 32) + beta * (D // 64) + blk // 2


def dim_tile_position(d, kb, D):
    """Byte of row d and key block kb (0..3) in one V^T scale tile."""
    return (32 * (kb % 2) + d % 32) * (D // 16) + (kb // 2) * (D // 32) + d // 32


def _unpermute_k_scales(ks, S, D, bits):
    sk = ks.shape[0] * 128
    nb = D // 32
    pos = np.array([[key_tile_position(r % 128, b, D, bits) for b in range(nb)] for r in range(128)])
    out = np.empty((sk, nb), np.uint8)
    for t in range(ks.shape[0]):
        out[128 * t:128 * t + 128] = ks[t][pos]
    return out


def _unpermute_v_scales(vs, D):
    n_tiles = vs.shape[0]
    pos = np.array([[dim_tile_position(d, kb, D) for kb in range(4)] for d in range(D)])
    out = np.empty((D, 4 * n_tiles), np.uint8)
    for t in range(n_tiles):
        out[:, 4 * t:4 * t + 4] = vs[t][pos]
    return out


def _check_head(got, qh, kh, vh, fmt, b, h):
    S, D = qh.shape
    bits = BITS[fmt]
    sk = (S + 127) // 128 * 128
    g = {n: t[b, h].cpu().numpy() for n, t in got.items()}
    # Q'^: the prologue's quantisation of q' = fp32(q * c)
    qc, qs = O.mx_quantize(prescale_q(qh), fmt)
    assert np.array_equal(g["q_codes"], O.pack_codes(qc, fmt)), "q codes"
    raised = np.where(qs == 255, 255, np.minimum(qs.astype(np.int64) + 23, 254)).astype(np.uint8)
    assert np.array_equal(g["q_scales"], raised), "q scales"
    # K^: rows along D, padding rows zero
    kc, ks = O.mx_quantize(kh, fmt)
    assert np.array_equal(g["k_codes"][:S], O.pack_codes(kc, fmt)), "k codes"
    assert not g["k_codes"][S:].any()
    kso = _unpermute_k_scales(g["k_scales"], S, D, bits)
    assert np.array_equal(kso[:S], ks), "k scales"
    assert not kso[S:].any()
    # V^T: blocks along the keys, transposed, padding keys zero
    vc, vs = O.mx_quantize(np.ascontiguousarray(vh.T), fmt)
    nbytes = vc.shape[1] * bits // 8
    assert np.array_equal(g["v_codes"][:, :nbytes], O.pack_codes(vc, fmt)), "v codes"
    assert not g["v_codes"][:, nbytes:].any()
    vso = _unpermute_v_scales(g["v_scales"], D)
    assert np.array_equal(vso[:, :vs.shape[1]], vs), "v scales"
    assert not vso[:, vs.shape[1]:].any()


@pytest.mark.parametrize("fmt", ["e4m3", "e2m3", "e2m1"])
@pytest.mark.parametrize("D", [64, 128])
def test_operands_bit_exact_small(fmt, D):
    import torch
    import softmax_mx_quantize_amd as fsa
    S = 333
    announce("operands", fmt, D, S)
    rng = np.random.default_rng(3)
    q, k, v = (W.bf16_bits_to_f64(W.random_bf16((2, 2, S, D), seed, 1.7)) for seed in (51, 52, 53))
    # rows that reach the scale clamps and saturation: all zero, tiny, huge,
    # a lone large element among small ones
    q[0, 0, 5] = 0.0
    k[0, 1, 7] = 0.0
    q[1, 0, 9] *= 1e-36
    k[1, 1, 200] *= 1e-37
    v[0, 0, 40:72, 3] *= 1e30
    q[1, 1, 100, 17] = 3.0e4
    k[0, 0, 300, 63] = -2.5e5
    q, k, v = (W.f32_to_bf16_bits(x.astype(np.float32)) for x in (q, k, v))
    got = fsa.debug_operands(to_dev(q), to_dev(k), to_dev(v), fmt)
    torch.cuda.synchronize()
    for b in range(2):
        for h in range(2):
            _check_head(got, *(W.bf16_bits_to_f64(x[b, h]) for x in (q, k, v)), fmt, b, h)


@pytest.mark.parametrize("name", ["video_dit_e4m3", "video_dit_e2m3", "video_dit_e2m1"])
def test_operands_bit_exact_full_size(name):
    import torch
    import softmax_mx_quantize_amd as fsa
    from gpu_helpers import workload_tensors
    w = W.WORKLOADS[name]
    announce("operands full size", name)
    q, k, v = workload_tensors(w)
    got = fsa.debug_operands(to_dev(q), to_dev(k), to_dev(v), w.head_fmts[0])
    torch.cuda.synchronize()
    for h in (0, 39):
        _check_head(got, *(W.bf16_bits_to_f64(x[0, h]) for x in (q, k, v)), w.head_fmts[0], 0, h)
