"""Python binding of libfsa (fused-softmax MX attention for MI355X / gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libfsa.so``.  PyTorch supplies device memory and streams.  The
C ABI and its contract are declared in ``include/fsa.h``; the functions here
have the same names without the ``fsa_`` prefix.

Importing the package loads the shared library and fails loudly if it has not
been built (``python softmax_mx_quantize_amd/build.py``).
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple, Union

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("FSA_LIB_PATH") or os.path.join(_HERE, "libfsa.so")

FMT = {"e4m3": 0, "e2m3": 1, "e2m1": 2}
BITS = {0: 8, 1: 6, 2: 4}
STATUS = {0: "FSA_OK", -1: "FSA_ERR_INVALID_ARG", -2: "FSA_ERR_UNSUPPORTED",
          -3: "FSA_ERR_HIP", -4: "FSA_ERR_NO_MEMORY", -5: "FSA_ERR_TOO_LARGE"}


class FsaError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__("%s failed: %s (%s)" % (what, strerror(status), STATUS.get(status, status)))
        self.status = status


class Layout(ctypes.Structure):
    """Mirror of ``fsa_layout``: element strides (batch, head, row) per tensor."""
    _fields_ = [("q", ctypes.c_int64 * 3), ("k", ctypes.c_int64 * 3),
                ("v", ctypes.c_int64 * 3), ("out", ctypes.c_int64 * 3)]


class Options(ctypes.Structure):
    """Mirror of ``fsa_options``."""
    _fields_ = [
        ("guess_bias", ctypes.c_float),
        ("row_kappa", ctypes.c_void_p),
        ("row_max_guess", ctypes.c_void_p),
        ("event_after_quantize", ctypes.c_void_p),
        ("head_fmt", ctypes.POINTER(ctypes.c_int)),
        ("layout", ctypes.POINTER(Layout)),
        ("p_variant", ctypes.c_int),
        ("skip_fallback_pass", ctypes.c_int),
    ]


# fsa_p_variant
P_VARIANT = {"block": 0, "row": 1, "e4m3": 2, "affine": 3, "exact_exp": 4, "e3m2": 5}


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError("libfsa.so is not built: run `python softmax_mx_quantize_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.fsa_quantize_mx.argtypes = [vp, vp, vp, i64, i64, i64, i32, i32, vp]
    lib.fsa_quantize_mx.restype = i32
    lib.fsa_attention_fwd.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp]
    lib.fsa_attention_fwd.restype = i32
    lib.fsa_attention_fwd_ex.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                         ctypes.POINTER(Options), vp]
    lib.fsa_attention_fwd_ex.restype = i32
    lib.fsa_attention_fwd_noalloc.argtypes = lib.fsa_attention_fwd_ex.argtypes
    lib.fsa_attention_fwd_noalloc.restype = i32
    lib.fsa_attention_bf16_ref.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, vp]
    lib.fsa_attention_bf16_ref.restype = i32
    lib.fsa_strerror.argtypes = [i32]
    lib.fsa_strerror.restype = ctypes.c_char_p
    lib.fsa_release_workspace.argtypes = []
    lib.fsa_release_workspace.restype = i32
    lib.fsa_debug_operands.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp]
    lib.fsa_debug_operands.restype = i32
    return lib


lib = _load()

EXPORTS = ("fsa_quantize_mx", "fsa_attention_fwd", "fsa_attention_fwd_ex",
           "fsa_attention_bf16_ref", "fsa_strerror", "fsa_release_workspace",
           "fsa_debug_operands", "fsa_attention_fwd_noalloc")


def strerror(status: int) -> str:
    return lib.fsa_strerror(int(status)).decode()


def _fmt_id(fmt: Union[str, int]) -> int:
    return FMT[fmt] if isinstance(fmt, str) else int(fmt)


def _stream(t) -> int:
    import torch
    return torch.cuda.current_stream(t.device).cuda_stream


def _check(st: int, what: str) -> None:
    if st != 0:
        raise FsaError(st, what)


def _bf16_cuda(*ts) -> None:
    import torch
    for t in ts:
        if not (t.is_cuda and t.dtype == torch.bfloat16 and t.is_contiguous()):
            raise ValueError("expected contiguous bf16 CUDA tensors")


def _bf16_rows(*ts) -> None:
    """bf16 CUDA tensors [B, H, S, D] whose rows are contiguous (strided
    views, e.g. of a [B, S, H, D] tensor, are fine)."""
    import torch
    for t in ts:
        if not (t.is_cuda and t.dtype == torch.bfloat16 and t.dim() == 4 and t.stride(-1) == 1):
            raise ValueError("expected bf16 CUDA tensors [B, H, S, D] with contiguous rows")


def _layout(q, k, v, out):
    """An fsa_layout when any tensor is not contiguous [B, H, S, D]."""
    if all(t.is_contiguous() for t in (q, k, v, out)):
        return None
    lay = Layout()
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        getattr(lay, name)[:] = [t.stride(0), t.stride(1), t.stride(2)]
    return lay


def _out_like(out, q):
    """A caller's output tensor must match q in shape, dtype and device,
    with contiguous rows (the kernels write whole bf16 rows); a new
    contiguous one otherwise."""
    import torch
    if out is None:
        return torch.empty(q.shape, dtype=q.dtype, device=q.device)
    _bf16_rows(out)
    if out.shape != q.shape or out.device != q.device:
        raise ValueError("out must be a bf16 tensor of q's shape on q's device, rows contiguous")
    return out


def quantize_mx(x, fmt: Union[str, int], block_along_rows: bool = False):
    """MX-quantise a bf16 [batch, rows, cols] tensor; returns (codes, scales) uint8."""
    import torch
    _bf16_cuda(x)
    if x.dim() == 2:
        x = x.unsqueeze(0)
    batch, rows, cols = x.shape
    f = _fmt_id(fmt)
    valid, out_rows = (rows, cols) if block_along_rows else (cols, rows)
    nb = (valid + 31) // 32
    codes = torch.empty((batch, out_rows, nb * 4 * BITS.get(f, 8)), dtype=torch.uint8, device=x.device)
    scales = torch.empty((batch, out_rows, nb), dtype=torch.uint8, device=x.device)
    _check(lib.fsa_quantize_mx(x.data_ptr(), codes.data_ptr(), scales.data_ptr(), batch, rows,
                               cols, f, int(block_along_rows), _stream(x)), "fsa_quantize_mx")
    return codes, scales


def attention_fwd(q, k, v, fmt: Union[str, int] = "e4m3", causal: bool = False, *,
                  guess_bias: float = 0.0, head_fmt: Optional[Sequence[Union[str, int]]] = None,
                  return_rows: bool = False, event_after_quantize=None, out=None,
                  no_alloc: bool = False, p_variant: Union[str, int] = "block",
                  skip_fallback_pass: bool = False):
    """Fused-softmax attention; q, k, v bf16 [B, H, S, D] CUDA tensors
    (strided views with contiguous rows are passed with their strides).

    With ``return_rows`` also returns the per-row fallback offsets (int32)
    and frozen maxima (float32), each [B, H, S].  ``no_alloc`` calls
    ``fsa_attention_fwd_noalloc`` (the library allocates nothing; the
    tensors here are still torch's).  ``p_variant`` picks the P~ variant
    (``fsa_p_variant``: "block", "row", "e4m3", "affine", "exact_exp", "e3m2").
    """
    import torch
    _bf16_rows(q, k, v)
    B, H, S, D = q.shape
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must have the same shape")
    if k.device != q.device or v.device != q.device:
        raise ValueError("q, k, v must be on one device")
    out = _out_like(out, q)
    opt = Options()
    opt.guess_bias = float(guess_bias)
    opt.p_variant = P_VARIANT[p_variant] if isinstance(p_variant, str) else int(p_variant)
    opt.skip_fallback_pass = int(bool(skip_fallback_pass))
    kappa = mg = None
    if return_rows:
        kappa = torch.empty((B, H, S), dtype=torch.int32, device=q.device)
        mg = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
        opt.row_kappa = kappa.data_ptr()
        opt.row_max_guess = mg.data_ptr()
    if event_after_quantize is not None:
        opt.event_after_quantize = event_after_quantize.cuda_event
    lay = _layout(q, k, v, out)
    if lay is not None:
        opt.layout = ctypes.pointer(lay)
    hf = None
    if head_fmt is not None:
        if len(head_fmt) != H:
            raise ValueError("head_fmt needs one entry per head")
        hf = (ctypes.c_int * H)(*[_fmt_id(x) for x in head_fmt])
        opt.head_fmt = hf
    fn = lib.fsa_attention_fwd_noalloc if no_alloc else lib.fsa_attention_fwd_ex
    st = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, H, S, D, _fmt_id(fmt),
            int(causal), ctypes.byref(opt), _stream(q))
    _check(st, "fsa_attention_fwd_noalloc" if no_alloc else "fsa_attention_fwd")
    if return_rows:
        return out, kappa, mg
    return out


def attention_bf16_ref(q, k, v, causal: bool = False, out=None):
    """Plain BF16 flash attention (the in-house baseline); bf16 [B, H, S, D]."""
    import torch
    _bf16_cuda(q, k, v)
    B, H, S, D = q.shape
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must have the same shape")
    if k.device != q.device or v.device != q.device:
        raise ValueError("q, k, v must be on one device")
    out = _out_like(out, q)
    _bf16_cuda(out)                 # the baseline writes contiguous [B, H, S, D]
    _check(lib.fsa_attention_bf16_ref(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                      B, H, S, D, int(causal), _stream(q)), "fsa_attention_bf16_ref")
    return out


def debug_operands(q, k, v, fmt: Union[str, int] = "e4m3"):
    """The MX operands as the attention kernels consume them (layouts in
    ``include/fsa.h``): a dict of uint8 tensors q_codes, q_scales, k_codes,
    k_scales (key-tile order), v_codes (transposed), v_scales (tile order)."""
    import torch
    _bf16_cuda(q, k, v)
    B, H, S, D = q.shape
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must have the same shape")
    f = _fmt_id(fmt)
    bits = BITS.get(f, 8)
    sk = (S + 127) // 128 * 128
    u8 = lambda *shape: torch.empty(shape, dtype=torch.uint8, device=q.device)
    out = {"q_codes": u8(B, H, S, D * bits // 8), "q_scales": u8(B, H, S, D // 32),
           "k_codes": u8(B, H, sk, D * bits // 8), "k_scales": u8(B, H, sk // 128, 128 * D // 32),
           "v_codes": u8(B, H, D, sk * bits // 8), "v_scales": u8(B, H, sk // 128, 4 * D)}
    p = {n: t.data_ptr() for n, t in out.items()}
    _check(lib.fsa_debug_operands(q.data_ptr(), k.data_ptr(), v.data_ptr(), B, H, S, D, f,
                                  p["q_codes"], p["q_scales"], p["k_codes"], p["k_scales"],
                                  p["v_codes"], p["v_scales"], _stream(q)), "fsa_debug_operands")
    return out


def release_workspace() -> None:
    _check(lib.fsa_release_workspace(), "fsa_release_workspace")
