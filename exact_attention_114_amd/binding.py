"""ctypes binding over the C ABI of libfa.so (declared in include/fa.h).

Argument marshalling only: tensors are checked for device, dtype, layout and
shape, outputs (and the backward's workspace) are allocated when the caller
does not pass them, and every step of the computation runs in the HIP
kernels behind ``fa_fwd`` and ``fa_bwd``. There is no fallback: when the
library is missing the first call raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

LIB_NAME = "libfa.so"

FA_F16, FA_BF16, FA_F32 = 0, 1, 2
FA_OK, FA_ERR_NULLPTR, FA_ERR_SHAPE, FA_ERR_UNSUPPORTED, FA_ERR_ALIGN, FA_ERR_HIP, FA_ERR_SCRATCH = range(7)
NOALLOC_SCRATCH_BYTES = 64 << 20  # FA_NOALLOC_SCRATCH_BYTES

# Every function include/fa.h declares, with its ctypes signature.
SIGNATURES = {
    "fa_fwd": (ctypes.c_int, [ctypes.c_void_p] * 5 + [ctypes.c_int64] * 5
               + [ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]),
    "fa_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "fa_last_hip_error": (ctypes.c_int, []),
    "fa_fwd_tile": (ctypes.c_int, [ctypes.c_int64] * 5 + [ctypes.c_int, ctypes.c_int,
                                                          ctypes.POINTER(ctypes.c_int),
                                                          ctypes.POINTER(ctypes.c_int),
                                                          ctypes.POINTER(ctypes.c_int64)]),
    "fa_bwd": (ctypes.c_int, [ctypes.c_void_p] * 10 + [ctypes.c_int64] * 5
               + [ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]),
    "fa_bwd_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int64] * 4),
    "fa_fwd_ex": (ctypes.c_int, [ctypes.c_void_p] * 5 + [ctypes.c_int64] * 6 + [ctypes.c_float]
                  + [ctypes.c_int64] * 2 + [ctypes.c_int, ctypes.c_int, ctypes.c_void_p]),
    "fa_bwd_ex": (ctypes.c_int, [ctypes.c_void_p] * 10 + [ctypes.c_int64] * 6 + [ctypes.c_float]
                  + [ctypes.c_int64] * 2 + [ctypes.c_int, ctypes.c_int, ctypes.c_void_p]),
    "fa_fwd_split": (ctypes.c_int, [ctypes.c_void_p] * 6 + [ctypes.c_int64] * 6 + [ctypes.c_float]
                     + [ctypes.c_int64] * 2 + [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]),
    "fa_fwd_split_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int64] * 5 + [ctypes.c_int]),
    "fa_fwd_fp8": (ctypes.c_int, [ctypes.c_void_p] * 5 + [ctypes.c_float] * 3 + [ctypes.c_int64] * 6
                   + [ctypes.c_float] + [ctypes.c_int64] * 2 + [ctypes.c_void_p]),
    "fa_fwd_dropout": (ctypes.c_int, [ctypes.c_void_p] * 5 + [ctypes.c_int64] * 6 + [ctypes.c_float]
                       + [ctypes.c_int64] * 2 + [ctypes.c_float, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int,
                                                 ctypes.c_int, ctypes.c_void_p]),
    "fa_bwd_dropout": (ctypes.c_int, [ctypes.c_void_p] * 10 + [ctypes.c_int64] * 6 + [ctypes.c_float]
                       + [ctypes.c_int64] * 2 + [ctypes.c_float, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int,
                                                 ctypes.c_int, ctypes.c_void_p]),
    "fa_fwd_float_mask": (ctypes.c_int, [ctypes.c_void_p] * 6 + [ctypes.c_int] + [ctypes.c_int64] * 9
                          + [ctypes.c_float] + [ctypes.c_int64] * 2 + [ctypes.c_int, ctypes.c_int, ctypes.c_void_p]),
    "fa_bwd_float_mask": (ctypes.c_int, [ctypes.c_void_p] * 11 + [ctypes.c_int] + [ctypes.c_int64] * 9
                          + [ctypes.c_float] + [ctypes.c_int64] * 2 + [ctypes.c_int, ctypes.c_int, ctypes.c_void_p]),
    "fa_fwd_split_noalloc": (ctypes.c_int, [ctypes.c_void_p] * 5 + [ctypes.c_int64] * 6 + [ctypes.c_float]
                             + [ctypes.c_int64] * 2 + [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]),
    "fa_fwd_mask_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int64] * 5 + [ctypes.c_int] + [ctypes.c_int64] * 2),
    "fa_bwd_mask_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int64] * 7),
    "fa_bwd_mask": (ctypes.c_int, [ctypes.c_void_p] * 11 + [ctypes.c_int64] * 9 + [ctypes.c_float]
                    + [ctypes.c_int64] * 2 + [ctypes.c_int, ctypes.c_int, ctypes.c_void_p]),
    "fa_fwd_mask": (ctypes.c_int, [ctypes.c_void_p] * 6 + [ctypes.c_int64] * 3 + [ctypes.c_void_p]
                    + [ctypes.c_int64] * 6 + [ctypes.c_float] + [ctypes.c_int64] * 2
                    + [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]),
}

_lib = None


class FaError(RuntimeError):
    """An fa_status other than FA_OK, or a missing library."""

    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def library_path() -> str:
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), LIB_NAME)


def load_library() -> ctypes.CDLL:
    """Open libfa.so next to this file (raises FaError if it was never built)."""
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            raise FaError(-1, f"{path} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")
        lib = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def status_str(status: int) -> str:
    return load_library().fa_status_str(status).decode()


def _check(status: int) -> None:
    if status != FA_OK:
        lib = load_library()
        msg = lib.fa_status_str(status).decode()
        if status == FA_ERR_HIP:
            msg += f" (hipError_t {lib.fa_last_hip_error()})"
        raise FaError(status, msg)


def fwd_raw(q: int, k: int, v: int, o: int, lse: int, B: int, Hq: int, Hkv: int, N: int, d: int,
            scale: float, causal: bool, in_dtype: int, out_dtype: int, stream: int = 0) -> int:
    """Call fa_fwd with raw device addresses; returns the fa_status code."""
    return load_library().fa_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, float(scale), int(causal),
                                 in_dtype, out_dtype, stream)


def fwd_ex_raw(q: int, k: int, v: int, o: int, lse: int, B: int, Hq: int, Hkv: int, Nq: int, Nk: int, d: int,
               scale: float, left: int, right: int, in_dtype: int, out_dtype: int, stream: int = 0) -> int:
    """Call fa_fwd_ex with raw device addresses; returns the fa_status code."""
    return load_library().fa_fwd_ex(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, float(scale), left, right,
                                    in_dtype, out_dtype, stream)


def fwd_split_raw(q: int, k: int, v: int, o: int, lse: int, ws: int, B: int, Hq: int, Hkv: int, Nq: int, Nk: int,
                  d: int, scale: float, left: int, right: int, n_splits: int, in_dtype: int, out_dtype: int,
                  stream: int = 0) -> int:
    """Call fa_fwd_split with raw device addresses; returns the fa_status code."""
    return load_library().fa_fwd_split(q, k, v, o, lse, ws, B, Hq, Hkv, Nq, Nk, d, float(scale), left, right,
                                       n_splits, in_dtype, out_dtype, stream)


def fwd_split_noalloc_raw(q: int, k: int, v: int, o: int, lse: int, B: int, Hq: int, Hkv: int, Nq: int, Nk: int,
                          d: int, scale: float, left: int, right: int, n_splits: int, in_dtype: int, out_dtype: int,
                          stream: int = 0) -> int:
    """Call fa_fwd_split_noalloc (split partials in the library's static scratch) with raw device
    addresses; returns the fa_status code."""
    return load_library().fa_fwd_split_noalloc(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, float(scale), left, right,
                                               n_splits, in_dtype, out_dtype, stream)


def fwd_dropout_raw(q: int, k: int, v: int, o: int, lse: int, B: int, Hq: int, Hkv: int, Nq: int, Nk: int, d: int,
                    scale: float, left: int, right: int, keep_prob: float, seed: int, offset: int, in_dtype: int,
                    out_dtype: int, stream: int = 0) -> int:
    """Call fa_fwd_dropout with raw device addresses; returns the fa_status code."""
    return load_library().fa_fwd_dropout(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, float(scale), left, right,
                                         float(keep_prob), int(seed) & (2 ** 64 - 1), int(offset) & 0xFFFFFFFF,
                                         in_dtype, out_dtype, stream)


def fwd_fp8_raw(q: int, k: int, v: int, o: int, lse: int, descale_q: float, descale_k: float, descale_v: float,
                B: int, Hq: int, Hkv: int, Nq: int, Nk: int, d: int, scale: float, left: int, right: int,
                stream: int = 0) -> int:
    """Call fa_fwd_fp8 with raw device addresses; returns the fa_status code."""
    return load_library().fa_fwd_fp8(q, k, v, o, lse, float(descale_q), float(descale_k), float(descale_v), B, Hq,
                                     Hkv, Nq, Nk, d, float(scale), left, right, stream)


def fwd_fp8(q, k, v, descale_q: float, descale_k: float, descale_v: float, *, scale: Optional[float] = None,
            causal: bool = False, window=None, out=None, lse=None, stream=None):
    """fp8 (OCP e4m3) attention forward: returns (O float32, LSE float32).

    q [B, Hq, Nq, d], k and v [B, Hkv, Nk, d]: contiguous uint8 (or torch.float8_e4m3fn) CUDA
    tensors of e4m3 bytes; each tensor's real values are its bytes' values times its descale.
    scale defaults to 1/sqrt(d); causal and window as for ``fwd``.
    """
    import torch

    fp8 = getattr(torch, "float8_e4m3fn", None)
    for t in (q, k, v):
        if t.dtype not in (torch.uint8,) + ((fp8,) if fp8 is not None else ()):
            raise FaError(FA_ERR_UNSUPPORTED, "q, k, v must hold e4m3 bytes (uint8 or float8_e4m3fn)")
        if not t.is_cuda or not t.is_contiguous() or t.dim() != 4:
            raise FaError(FA_ERR_SHAPE, "q, k, v must be contiguous 4-D GPU tensors")
    B, Hq, N, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != d:
        raise FaError(FA_ERR_SHAPE, f"k/v shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    Hkv, Nk = k.shape[1], k.shape[2]
    left, right = _edges(causal, window)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, Hq, N, d), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    if out.shape != (B, Hq, N, d) or out.dtype != torch.float32 or not out.is_contiguous():
        raise FaError(FA_ERR_SHAPE, "out must be a contiguous float32 [B, Hq, N, d] tensor")
    if lse.shape != (B, Hq, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise FaError(FA_ERR_SHAPE, "lse must be a contiguous float32 [B, Hq, N] tensor")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    _check(fwd_fp8_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), descale_q,
                       descale_k, descale_v, B, Hq, Hkv, N, Nk, d, scale, left, right, stream.cuda_stream))
    return out, lse


def fwd_mask_raw(q: int, k: int, v: int, o: int, lse: int, mask: int, m_sb: int, m_sh: int, m_ld: int, ws: int,
                 B: int, Hq: int, Hkv: int, Nq: int, Nk: int, d: int, scale: float, left: int, right: int,
                 n_splits: int, in_dtype: int, out_dtype: int, stream: int = 0) -> int:
    """Call fa_fwd_mask with raw device addresses; returns the fa_status code."""
    return load_library().fa_fwd_mask(q, k, v, o, lse, mask, m_sb, m_sh, m_ld, ws, B, Hq, Hkv, Nq, Nk, d,
                                      float(scale), left, right, n_splits, in_dtype, out_dtype, stream)


def bwd_mask_raw(q: int, k: int, v: int, o: int, lse: int, dout: int, dq: int, dk: int, dv: int, ws: int,
                 mask: int, m_sb: int, m_sh: int, m_ld: int, B: int, Hq: int, Hkv: int, Nq: int, Nk: int, d: int,
                 scale: float, left: int, right: int, in_dtype: int, o_dtype: int, stream: int = 0) -> int:
    """Call fa_bwd_mask with raw device addresses; returns the fa_status code."""
    return load_library().fa_bwd_mask(q, k, v, o, lse, dout, dq, dk, dv, ws, mask, m_sb, m_sh, m_ld, B, Hq, Hkv,
                                      Nq, Nk, d, float(scale), left, right, in_dtype, o_dtype, stream)


def fwd_float_mask_raw(q: int, k: int, v: int, o: int, lse: int, mask: int, mask_dtype: int, m_sb: int, m_sh: int,
                       m_ld: int, B: int, Hq: int, Hkv: int, Nq: int, Nk: int, d: int, scale: float, left: int,
                       right: int, in_dtype: int, out_dtype: int, stream: int = 0) -> int:
    """Call fa_fwd_float_mask with raw device addresses; returns the fa_status code."""
    return load_library().fa_fwd_float_mask(q, k, v, o, lse, mask, mask_dtype, m_sb, m_sh, m_ld, B, Hq, Hkv, Nq, Nk,
                                            d, float(scale), left, right, in_dtype, out_dtype, stream)


def bwd_float_mask_raw(q: int, k: int, v: int, o: int, lse: int, dout: int, dq: int, dk: int, dv: int, ws: int,
                       mask: int, mask_dtype: int, m_sb: int, m_sh: int, m_ld: int, B: int, Hq: int, Hkv: int,
                       Nq: int, Nk: int, d: int, scale: float, left: int, right: int, in_dtype: int, o_dtype: int,
                       stream: int = 0) -> int:
    """Call fa_bwd_float_mask with raw device addresses; returns the fa_status code."""
    return load_library().fa_bwd_float_mask(q, k, v, o, lse, dout, dq, dk, dv, ws, mask, mask_dtype, m_sb, m_sh,
                                            m_ld, B, Hq, Hkv, Nq, Nk, d, float(scale), left, right, in_dtype,
                                            o_dtype, stream)


def float_mask_args(mask, B: int, Hq: int, Nq: int, Nk: int) -> Tuple[int, int, int, int]:
    """(dtype code, batch, head, row strides in elements) of a [B or 1, Hq or 1, Nq, Nk] float16 or
    float32 additive mask tensor, a size-1 batch or head axis shared (stride 0). Rows must be
    contiguous with a row stride that is a multiple of 4 elements (pad the key axis)."""
    import torch

    code = {torch.float16: FA_F16, torch.float32: FA_F32}.get(mask.dtype)
    if code is None:
        raise FaError(FA_ERR_UNSUPPORTED, "a float mask must be float16 or float32")
    if mask.dim() != 4 or mask.shape[2] != Nq or mask.shape[3] != Nk or mask.shape[0] not in (1, B) \
            or mask.shape[1] not in (1, Hq):
        raise FaError(FA_ERR_SHAPE, f"mask shape {tuple(mask.shape)} is not [B or 1, Hq or 1, {Nq}, {Nk}]")
    if mask.stride(3) != 1 or mask.stride(2) % 4 != 0:
        raise FaError(FA_ERR_ALIGN, "mask rows must be contiguous with a row stride that is a multiple of 4 "
                                    "elements (pad the key axis)")
    sb = mask.stride(0) if mask.shape[0] > 1 else 0
    sh = mask.stride(1) if mask.shape[1] > 1 else 0
    return code, sb, sh, mask.stride(2)


def is_float_mask(mask) -> bool:
    import torch

    return mask is not None and mask.dtype in (torch.float16, torch.float32)


def mask_strides(mask, B: int, Hq: int, Nq: int, Nk: int) -> Tuple[int, int, int]:
    """(batch, head, row) byte strides of a [B or 1, Hq or 1, Nq, Nk] bool or uint8 mask tensor,
    a size-1 batch or head axis shared (stride 0). Rows must be contiguous and 4-byte aligned."""
    import torch

    if mask.dtype not in (torch.bool, torch.uint8):
        raise FaError(FA_ERR_UNSUPPORTED, "mask must be bool or uint8 (nonzero hides the key)")
    if mask.dim() != 4 or mask.shape[2] != Nq or mask.shape[3] != Nk or mask.shape[0] not in (1, B) \
            or mask.shape[1] not in (1, Hq):
        raise FaError(FA_ERR_SHAPE, f"mask shape {tuple(mask.shape)} is not [B or 1, Hq or 1, {Nq}, {Nk}]")
    if mask.stride(3) != 1 or mask.stride(2) % 4 != 0:
        raise FaError(FA_ERR_ALIGN, "mask rows must be contiguous with a row stride that is a multiple of 4 bytes "
                                    "(pad the key axis)")
    sb = mask.stride(0) if mask.shape[0] > 1 else 0
    sh = mask.stride(1) if mask.shape[1] > 1 else 0
    return sb, sh, mask.stride(2)


def split_workspace_bytes(B: int, Hq: int, Nq: int, Nk: int, d: int, n_splits: int) -> int:
    """Bytes of workspace fa_fwd_split needs (0: it would not split)."""
    return int(load_library().fa_fwd_split_workspace_bytes(B, Hq, Nq, Nk, d, n_splits))


def mask_workspace_bytes(B: int, Hq: int, Nq: int, Nk: int, d: int, n_splits: int, mask_b_stride: int,
                         mask_h_stride: int) -> int:
    """Bytes of workspace fa_fwd_mask needs for a mask with these batch and head strides
    (0: shared along that axis); 0 for sizes it rejects."""
    return int(load_library().fa_fwd_mask_workspace_bytes(B, Hq, Nq, Nk, d, n_splits, mask_b_stride,
                                                           mask_h_stride))


def bwd_mask_workspace_bytes(B: int, Hq: int, Nq: int, Nk: int, d: int, mask_b_stride: int,
                             mask_h_stride: int) -> int:
    """Bytes of workspace fa_bwd_mask needs for a mask with these batch and head strides
    (0: shared along that axis); 0 for sizes it rejects."""
    return int(load_library().fa_bwd_mask_workspace_bytes(B, Hq, Nq, Nk, d, mask_b_stride, mask_h_stride))


def _edges(causal: bool, window) -> Tuple[int, int]:
    """(left, right) band edges for the C ABI, -1 meaning unlimited."""
    if window is None:
        return -1, (0 if causal else -1)
    if causal:
        raise FaError(FA_ERR_SHAPE, "pass either causal=True or window=(left, right), not both")
    left, right = window
    return (-1 if left is None else int(left)), (-1 if right is None else int(right))


def tile(B: int, Hq: int, Hkv: int, N: int, d: int, causal: bool, in_dtype: int) -> Tuple[int, int, int]:
    """(query rows per work-group, keys per tile, work-group count) fa_fwd uses."""
    bm, bn, grid = ctypes.c_int(), ctypes.c_int(), ctypes.c_int64()
    _check(load_library().fa_fwd_tile(B, Hq, Hkv, N, d, int(bool(causal)), in_dtype,
                                      ctypes.byref(bm), ctypes.byref(bn), ctypes.byref(grid)))
    return bm.value, bn.value, grid.value


def fwd(q, k, v, *, scale: Optional[float] = None, causal: bool = False, window=None, out_dtype=None,
        out=None, lse=None, splits: Optional[int] = None, workspace=None, mask=None, dropout=None, stream=None):
    """Exact attention forward on the GPU: returns (O, LSE).

    q: [B, Hq, Nq, d], k and v: [B, Hkv, Nk, d], contiguous fp16, bf16 or fp32 CUDA
    tensors (on ROCm, HIP device tensors); fp32 inputs take fp32 O and neither split keys
    nor a mask. scale defaults to 1/sqrt(d);
    out_dtype defaults to float32 (or pass q.dtype); LSE is float32 [B, Hq, Nq].
    causal=True, or window=(left, right) (None for an unlimited edge), bands the
    keys as fa_fwd_ex does: query row i sees keys i + Nk - Nq - left ..
    i + Nk - Nq + right. Without a window, split or mask, and with as many keys as
    queries, the call is fa_fwd itself. splits (0 = automatic, or a chunk count up to 16) cuts each
    Q-tile's keys into chunks merged afterwards (fa_fwd_split); its workspace is
    allocated when not given. mask, a bool or uint8 [B or 1, Hq or 1, Nq, Nk] tensor whose
    nonzero entries hide keys (fa_fwd_mask), applies on top of the band; a float16 or
    float32 mask of that shape is added to the scaled scores instead (fa_fwd_float_mask,
    -inf hiding a key; no split keys). dropout=(keep_prob,
    seed, offset) drops probabilities with the Philox keep mask of fa_fwd_dropout (16-bit
    inputs, no split or mask). Runs on ``stream`` (a torch stream) or torch's current stream.
    """
    import torch

    if q.dtype not in (torch.float16, torch.bfloat16, torch.float32):
        raise FaError(FA_ERR_UNSUPPORTED, "q, k, v must be float16, bfloat16 or float32")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise FaError(FA_ERR_UNSUPPORTED, "q, k, v must share one dtype")
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise FaError(FA_ERR_SHAPE, "q, k, v must be 4-D [batch, heads, seq, head_dim]")
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise FaError(FA_ERR_UNSUPPORTED, "q, k, v must be GPU tensors")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise FaError(FA_ERR_SHAPE, "q, k, v must be contiguous")
    B, Hq, N, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != d:
        raise FaError(FA_ERR_SHAPE, f"k/v shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    Hkv, Nk = k.shape[1], k.shape[2]
    left, right = _edges(causal, window)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out_dtype is None:
        out_dtype = torch.float32
    in_code = {torch.float16: FA_F16, torch.bfloat16: FA_BF16, torch.float32: FA_F32}[q.dtype]
    if out_dtype == torch.float32:
        out_code = FA_F32
    elif out_dtype == q.dtype:
        out_code = in_code
    else:
        raise FaError(FA_ERR_UNSUPPORTED, "out_dtype must be float32 or the input dtype")
    if out is None:
        out = torch.empty((B, Hq, N, d), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    if out.shape != (B, Hq, N, d) or out.dtype != out_dtype or not out.is_contiguous():
        raise FaError(FA_ERR_SHAPE, "out must be a contiguous [B, Hq, N, d] tensor of out_dtype")
    if lse.shape != (B, Hq, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise FaError(FA_ERR_SHAPE, "lse must be a contiguous float32 [B, Hq, N] tensor")
    if out.device != q.device or lse.device != q.device or k.device != q.device or v.device != q.device:
        raise FaError(FA_ERR_SHAPE, "all tensors must be on one device")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    if dropout is not None:
        if mask is not None or splits is not None:
            raise FaError(FA_ERR_UNSUPPORTED, "dropout takes neither a mask nor split keys")
        keep_prob, seed, offset = dropout
        _check(fwd_dropout_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, Hq, Hkv,
                               N, Nk, d, scale, left, right, keep_prob, seed, offset, in_code, out_code,
                               stream.cuda_stream))
        return out, lse
    if is_float_mask(mask):
        if mask.device != q.device:
            raise FaError(FA_ERR_SHAPE, "mask must be on the inputs' device")
        if splits is not None:
            raise FaError(FA_ERR_UNSUPPORTED, "a float mask takes no split keys")
        mcode, sb, sh, ld = float_mask_args(mask, B, Hq, N, Nk)
        _check(fwd_float_mask_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                  mask.data_ptr(), mcode, sb, sh, ld, B, Hq, Hkv, N, Nk, d, scale, left, right,
                                  in_code, out_code, stream.cuda_stream))
        return out, lse
    if mask is not None:
        if mask.device != q.device:
            raise FaError(FA_ERR_SHAPE, "mask must be on the inputs' device")
        sb, sh, ld = mask_strides(mask, B, Hq, N, Nk)
        ns = 1 if splits is None else int(splits)
        need = mask_workspace_bytes(B, Hq, N, Nk, d, ns, sb, sh)
        if workspace is None:
            workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
        if workspace.device != q.device or workspace.numel() * workspace.element_size() < need:
            raise FaError(FA_ERR_SHAPE, f"workspace must hold {need} bytes on the inputs' device")
        _check(fwd_mask_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                            mask.data_ptr(), sb, sh, ld, workspace.data_ptr(), B, Hq, Hkv, N, Nk, d,
                            scale, left, right, ns, in_code, out_code, stream.cuda_stream))
        return out, lse
    if splits is not None:
        need = split_workspace_bytes(B, Hq, N, Nk, d, int(splits))
        if workspace is None:
            workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
        if workspace.device != q.device or workspace.numel() * workspace.element_size() < need:
            raise FaError(FA_ERR_SHAPE, f"workspace must hold {need} bytes on the inputs' device")
        _check(fwd_split_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                             workspace.data_ptr(), B, Hq, Hkv, N, Nk, d, scale, left, right, int(splits), in_code,
                             out_code, stream.cuda_stream))
        return out, lse
    if window is None and Nk == N:
        # plain or causal attention over one sequence: the boundary's own entry point
        _check(fwd_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                       B, Hq, Hkv, N, d, scale, causal, in_code, out_code, stream.cuda_stream))
        return out, lse
    _check(fwd_ex_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                      B, Hq, Hkv, N, Nk, d, scale, left, right, in_code, out_code, stream.cuda_stream))
    return out, lse


def bwd_raw(q: int, k: int, v: int, o: int, lse: int, dout: int, dq: int, dk: int, dv: int, ws: int,
            B: int, Hq: int, Hkv: int, N: int, d: int, scale: float, causal: bool, in_dtype: int,
            o_dtype: int, stream: int = 0) -> int:
    """Call fa_bwd with raw device addresses; returns the fa_status code."""
    return load_library().fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, ws, B, Hq, Hkv, N, d, float(scale),
                                 int(causal), in_dtype, o_dtype, stream)


def bwd_workspace_bytes(B: int, Hq: int, N: int, d: int) -> int:
    """Bytes of workspace fa_bwd needs (0 for sizes it rejects)."""
    return int(load_library().fa_bwd_workspace_bytes(B, Hq, N, d))


def bwd_ex_raw(q: int, k: int, v: int, o: int, lse: int, dout: int, dq: int, dk: int, dv: int, ws: int,
               B: int, Hq: int, Hkv: int, Nq: int, Nk: int, d: int, scale: float, left: int, right: int,
               in_dtype: int, o_dtype: int, stream: int = 0) -> int:
    """Call fa_bwd_ex with raw device addresses; returns the fa_status code."""
    return load_library().fa_bwd_ex(q, k, v, o, lse, dout, dq, dk, dv, ws, B, Hq, Hkv, Nq, Nk, d, float(scale),
                                    left, right, in_dtype, o_dtype, stream)


def bwd_dropout_raw(q: int, k: int, v: int, o: int, lse: int, dout: int, dq: int, dk: int, dv: int, ws: int,
                    B: int, Hq: int, Hkv: int, Nq: int, Nk: int, d: int, scale: float, left: int, right: int,
                    keep_prob: float, seed: int, offset: int, in_dtype: int, o_dtype: int, stream: int = 0) -> int:
    """Call fa_bwd_dropout with raw device addresses; returns the fa_status code."""
    return load_library().fa_bwd_dropout(q, k, v, o, lse, dout, dq, dk, dv, ws, B, Hq, Hkv, Nq, Nk, d, float(scale),
                                         left, right, float(keep_prob), int(seed) & (2 ** 64 - 1),
                                         int(offset) & 0xFFFFFFFF, in_dtype, o_dtype, stream)


def bwd(q, k, v, o, lse, dout, *, scale: Optional[float] = None, causal: bool = False, window=None,
        workspace=None, grads=None, mask=None, dropout=None, stream=None):
    """Gradients (dQ, dK, dV) of exact attention on the GPU, all float32.

    q, k, v as for ``fwd``; o and lse as ``fwd`` returned them (o float32 or
    the input dtype); dout: the gradient at o, [B, Hq, N, d] in the input
    dtype. causal and window as for ``fwd`` (k and v may have their own
    sequence length). The workspace (a uint8 CUDA tensor of at least
    ``bwd_workspace_bytes`` bytes, or ``bwd_mask_workspace_bytes`` with a mask) and the outputs (``grads``: contiguous
    float32 dq [B, Hq, N, d], dk and dv [B, Hkv, N, d]) are allocated when not
    given. mask, as for ``fwd`` (and the same one the forward used), goes to fa_bwd_mask
    (float16 or float32: fa_bwd_float_mask); dropout=(keep_prob, seed, offset), the
    forward's, to fa_bwd_dropout.
    Runs on ``stream`` or torch's current stream.
    """
    import torch

    if q.dtype not in (torch.float16, torch.bfloat16):
        raise FaError(FA_ERR_UNSUPPORTED, "q, k, v must be float16 or bfloat16")
    if k.dtype != q.dtype or v.dtype != q.dtype or dout.dtype != q.dtype:
        raise FaError(FA_ERR_UNSUPPORTED, "q, k, v and dout must share one dtype")
    if o.dtype not in (torch.float32, q.dtype) or lse.dtype != torch.float32:
        raise FaError(FA_ERR_UNSUPPORTED, "o must be float32 or the input dtype; lse float32")
    ts = (q, k, v, o, lse, dout)
    if any(not t.is_cuda for t in ts) or any(t.device != q.device for t in ts):
        raise FaError(FA_ERR_UNSUPPORTED, "all tensors must be on one GPU")
    if any(not t.is_contiguous() for t in ts):
        raise FaError(FA_ERR_SHAPE, "all tensors must be contiguous")
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise FaError(FA_ERR_SHAPE, "q, k, v must be 4-D [batch, heads, seq, head_dim]")
    B, Hq, N, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != d:
        raise FaError(FA_ERR_SHAPE, f"k/v shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    if o.shape != q.shape or dout.shape != q.shape or lse.shape != (B, Hq, N):
        raise FaError(FA_ERR_SHAPE, "o and dout must match q; lse must be [B, Hq, N]")
    Hkv, Nk = k.shape[1], k.shape[2]
    left, right = _edges(causal, window)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    in_code = FA_F16 if q.dtype == torch.float16 else FA_BF16
    o_code = FA_F32 if o.dtype == torch.float32 else in_code
    fmask = is_float_mask(mask)
    if mask is not None and mask.device != q.device:
        raise FaError(FA_ERR_SHAPE, "mask must be on the inputs' device")
    if fmask:
        mcode, sb, sh, ld = float_mask_args(mask, B, Hq, N, Nk)
        need = bwd_workspace_bytes(B, Hq, N, d)
    elif mask is not None:
        sb, sh, ld = mask_strides(mask, B, Hq, N, Nk)
        need = bwd_mask_workspace_bytes(B, Hq, N, Nk, d, sb, sh)
    else:
        need = bwd_workspace_bytes(B, Hq, N, d)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    if workspace.device != q.device or workspace.numel() * workspace.element_size() < need:
        raise FaError(FA_ERR_SHAPE, f"workspace must hold {need} bytes on the inputs' device")
    if grads is None:
        grads = (torch.empty((B, Hq, N, d), dtype=torch.float32, device=q.device),
                 torch.empty((B, Hkv, Nk, d), dtype=torch.float32, device=q.device),
                 torch.empty((B, Hkv, Nk, d), dtype=torch.float32, device=q.device))
    dq, dk, dv = grads
    for t, shp in ((dq, (B, Hq, N, d)), (dk, (B, Hkv, Nk, d)), (dv, (B, Hkv, Nk, d))):
        if t.shape != shp or t.dtype != torch.float32 or not t.is_contiguous() or t.device != q.device:
            raise FaError(FA_ERR_SHAPE, "grads must be contiguous float32 dq [B,Hq,Nq,d], dk and dv [B,Hkv,Nk,d]")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    if dropout is not None:
        if mask is not None:
            raise FaError(FA_ERR_UNSUPPORTED, "dropout takes no mask")
        keep_prob, seed, offset = dropout
        _check(bwd_dropout_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                               dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(), B,
                               Hq, Hkv, N, Nk, d, scale, left, right, keep_prob, seed, offset, in_code, o_code,
                               stream.cuda_stream))
        return dq, dk, dv
    if fmask:
        _check(bwd_float_mask_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                  dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(),
                                  mask.data_ptr(), mcode, sb, sh, ld, B, Hq, Hkv, N, Nk, d, scale, left, right,
                                  in_code, o_code, stream.cuda_stream))
        return dq, dk, dv
    if mask is not None:
        _check(bwd_mask_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), dout.data_ptr(),
                            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(), mask.data_ptr(), sb, sh,
                            ld, B, Hq, Hkv, N, Nk, d, scale, left, right, in_code, o_code, stream.cuda_stream))
        return dq, dk, dv
    _check(bwd_ex_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), dout.data_ptr(),
                      dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(), B, Hq, Hkv, N, Nk, d,
                      scale, left, right, in_code, o_code, stream.cuda_stream))
    return dq, dk, dv
