"""Python binding of libfa (exact tiled attention forward for MI355X).

Argument marshalling only: every step of the attention forward runs in the
HIP kernels behind the C ABI in ``include/fa.h``. PyTorch supplies device
memory and the stream; the library calls no torch operation.

The functions ``fa_fwd``, ``fa_fwd_fp32``, ``fa_fwd_window``, ``fa_fwd_bias``,
``fa_bwd``, ``fa_bwd_window``, ``fa_bwd_bias``, ``fa_fwd_splitkv``,
``fa_fwd_splitkv_noalloc``, ``fa_fwd_fp8``,
``fa_check_cu_seqlens``, ``fa_status_string``,
``fa_last_error`` and ``fa_version`` mirror the C entry points one to one
(raw integers and device addresses). ``attention_fwd`` is a convenience
wrapper that checks torch tensors, allocates O and LSE with torch and calls
``fa_fwd`` or ``fa_fwd_fp32`` on the current stream; ``attention_bwd`` does
the same for ``fa_bwd`` (dQ, dK, dV and the Dsum scratch).

Importing this package loads ``libfa.so`` from this directory and raises
ImportError if it is missing: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import math
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# FA_LIBRARY names another build of the same library (the host-sanitized
# one, say); by default the in-tree libfa.so is loaded.
LIB_PATH = os.environ.get("FA_LIBRARY") or os.path.join(_HERE, "libfa.so")

FA_OK = 0
FA_ERR_NULL = -1
FA_ERR_SHAPE = -2
FA_ERR_UNSUPPORTED = -3
FA_ERR_ARG = -4
FA_ERR_HIP = -5

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run `python exact_io_aware_63_amd/build.py` "
        "(hipcc, gfx950). There is no fallback path.")

_lib = ctypes.CDLL(LIB_PATH)

_FWD_ARGS = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
             ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
             ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.c_int, ctypes.c_void_p,
             ctypes.c_void_p]
_lib.fa_fwd.argtypes = _FWD_ARGS
_lib.fa_fwd.restype = ctypes.c_int
_lib.fa_fwd_fp32.argtypes = _FWD_ARGS
_lib.fa_fwd_fp32.restype = ctypes.c_int
_lib.fa_fwd_window.argtypes = ([ctypes.c_void_p] * 5 + [ctypes.c_int] * 6 +
                               [ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                ctypes.c_void_p, ctypes.c_void_p])
_lib.fa_fwd_window.restype = ctypes.c_int
_lib.fa_fwd_bias.argtypes = ([ctypes.c_void_p] * 5 + [ctypes.c_int] * 6 +
                             [ctypes.c_float, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64,
                              ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p])
_lib.fa_fwd_bias.restype = ctypes.c_int
_lib.fa_bwd.argtypes = ([ctypes.c_void_p] * 10 + [ctypes.c_int] * 6 +
                        [ctypes.c_float, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p])
_lib.fa_bwd.restype = ctypes.c_int
_lib.fa_bwd_bias.argtypes = ([ctypes.c_void_p] * 10 + [ctypes.c_int] * 6 +
                             [ctypes.c_float, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64,
                              ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p])
_lib.fa_bwd_bias.restype = ctypes.c_int
_lib.fa_bwd_window.argtypes = ([ctypes.c_void_p] * 10 + [ctypes.c_int] * 6 +
                               [ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                ctypes.c_void_p, ctypes.c_void_p])
_lib.fa_bwd_window.restype = ctypes.c_int
_lib.fa_fwd_splitkv.argtypes = ([ctypes.c_void_p] * 5 + [ctypes.c_int] * 6 +
                                [ctypes.c_float, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
                                 ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p])
_lib.fa_fwd_splitkv.restype = ctypes.c_int
_lib.fa_fwd_splitkv_noalloc.argtypes = ([ctypes.c_void_p] * 5 + [ctypes.c_int] * 6 +
                                        [ctypes.c_float, ctypes.c_int, ctypes.c_void_p,
                                         ctypes.c_int, ctypes.c_void_p])
_lib.fa_fwd_splitkv_noalloc.restype = ctypes.c_int
_lib.fa_fwd_fp8.argtypes = ([ctypes.c_void_p] * 5 + [ctypes.c_int] * 6 + [ctypes.c_float] * 4 +
                            [ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p])
_lib.fa_fwd_fp8.restype = ctypes.c_int
_lib.fa_fwd_fp8_workspace_bytes.argtypes = [ctypes.c_int] * 3
_lib.fa_fwd_fp8_workspace_bytes.restype = ctypes.c_size_t
_lib.fa_fwd_splitkv_workspace_bytes.argtypes = [ctypes.c_int] * 5
_lib.fa_fwd_splitkv_workspace_bytes.restype = ctypes.c_size_t
_lib.fa_fwd_splitkv_num_splits.argtypes = [ctypes.c_int] * 4
_lib.fa_fwd_splitkv_num_splits.restype = ctypes.c_int
_lib.fa_status_string.argtypes = [ctypes.c_int]
_lib.fa_status_string.restype = ctypes.c_char_p
_lib.fa_last_error.argtypes = []
_lib.fa_last_error.restype = ctypes.c_char_p
_lib.fa_check_cu_seqlens.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int]
_lib.fa_check_cu_seqlens.restype = ctypes.c_int
_lib.fa_version.argtypes = []
_lib.fa_version.restype = ctypes.c_int

EXPORTED = ("fa_fwd", "fa_fwd_fp32", "fa_fwd_window", "fa_fwd_bias", "fa_bwd", "fa_bwd_window",
            "fa_bwd_bias",
            "fa_fwd_splitkv", "fa_fwd_splitkv_workspace_bytes", "fa_fwd_splitkv_num_splits",
            "fa_fwd_splitkv_noalloc",
            "fa_fwd_fp8",
            "fa_fwd_fp8_workspace_bytes", "fa_check_cu_seqlens", "fa_status_string",
            "fa_last_error", "fa_version")


class FaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{fa_status_string(status)} ({detail})")
        self.status = status
        self.detail = detail


def fa_fwd(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, cu_seqlens, stream) -> int:
    """C ``fa_fwd``: pointers are integer device addresses (or 0 / None)."""
    return _lib.fa_fwd(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, int(causal),
                       cu_seqlens, stream)


def fa_fwd_fp32(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, cu_seqlens, stream) -> int:
    """C ``fa_fwd_fp32``: pointers are integer device addresses (or 0 / None)."""
    return _lib.fa_fwd_fp32(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, int(causal),
                            cu_seqlens, stream)


def fa_fwd_window(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, window_left, window_right,
                  cu_seqlens, stream) -> int:
    """C ``fa_fwd_window``: pointers are integer device addresses (or 0 / None)."""
    return _lib.fa_fwd_window(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, int(causal),
                              window_left, window_right, cu_seqlens, stream)


def fa_fwd_bias(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, bias, bias_stride_b,
                bias_stride_h, bias_stride_row, cu_seqlens, stream) -> int:
    """C ``fa_fwd_bias``: pointers are integer device addresses (or 0 / None)."""
    return _lib.fa_fwd_bias(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, int(causal), bias,
                            bias_stride_b, bias_stride_h, bias_stride_row, cu_seqlens, stream)


def bias_strides(bias, n_entries, hq, nq, nk):
    """Element strides (entry, head, row) of a bf16 bias tensor indexed
    [entry or 1, Hq or 1, >= Nq, >= Nk] with contiguous rows; an axis of
    extent 1 gets stride 0 (shared)."""
    import torch

    if bias.dtype != torch.bfloat16 or not bias.is_cuda or bias.dim() != 4:
        raise ValueError("bias must be a 4-D bfloat16 device tensor [entries|1, Hq|1, rows, cols]")
    if bias.shape[0] not in (1, n_entries) or bias.shape[1] not in (1, hq):
        raise ValueError(f"bias shape {tuple(bias.shape)} does not match {n_entries} entries "
                         f"and {hq} heads")
    if bias.shape[2] < nq or bias.shape[3] < nk:
        raise ValueError(f"bias shape {tuple(bias.shape)} does not cover Nq={nq}, Nk={nk}")
    if bias.stride(3) != 1 and bias.shape[3] > 1:
        raise ValueError("bias rows must be contiguous")
    sb = 0 if bias.shape[0] == 1 else bias.stride(0)
    sh = 0 if bias.shape[1] == 1 else bias.stride(1)
    return sb, sh, bias.stride(2)


def fa_bwd(q, k, v, o, do, lse, dq, dk, dv, dsum, B, Hq, Hkv, Nq, Nk, d, scale, causal,
           cu_seqlens, stream) -> int:
    """C ``fa_bwd``: pointers are integer device addresses (or 0 / None)."""
    return _lib.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, dsum, B, Hq, Hkv, Nq, Nk, d, scale,
                       int(causal), cu_seqlens, stream)


def fa_fwd_splitkv(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, seqlens_k, num_splits,
                   workspace, workspace_bytes, stream) -> int:
    """C ``fa_fwd_splitkv``: pointers are integer device addresses (or 0 / None)."""
    return _lib.fa_fwd_splitkv(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, int(causal),
                               seqlens_k, num_splits, workspace, workspace_bytes, stream)


FA_NOALLOC_SCRATCH_BYTES = 16 << 20


def fa_fwd_splitkv_noalloc(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, seqlens_k,
                           num_splits, stream) -> int:
    """C ``fa_fwd_splitkv_noalloc``: pointers are integer device addresses
    (or 0 / None); the split scratch is the library's own per-GPU array."""
    return _lib.fa_fwd_splitkv_noalloc(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale,
                                       int(causal), seqlens_k, num_splits, stream)


def fa_fwd_splitkv_workspace_bytes(B, Hq, Nq, d, num_splits) -> int:
    """C ``fa_fwd_splitkv_workspace_bytes``."""
    return _lib.fa_fwd_splitkv_workspace_bytes(B, Hq, Nq, d, num_splits)


def fa_fwd_splitkv_num_splits(B, Hkv, Nk, num_cus=0) -> int:
    """C ``fa_fwd_splitkv_num_splits``: a split count (>= 1) or a negative status."""
    return _lib.fa_fwd_splitkv_num_splits(B, Hkv, Nk, num_cus)


def fa_fwd_fp8(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, q_descale, k_descale, v_descale,
               causal, workspace, workspace_bytes, stream) -> int:
    """C ``fa_fwd_fp8``: pointers are integer device addresses (or 0 / None)."""
    return _lib.fa_fwd_fp8(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, q_descale, k_descale,
                           v_descale, int(causal), workspace, workspace_bytes, stream)


def fa_fwd_fp8_workspace_bytes(B, Hkv, Nk) -> int:
    """C ``fa_fwd_fp8_workspace_bytes``."""
    return _lib.fa_fwd_fp8_workspace_bytes(B, Hkv, Nk)


def attention_fwd_fp8(q, k, v, *, q_descale=1.0, k_descale=1.0, v_descale=1.0,
                      causal: bool = False, scale=None, stream=None):
    """FP8 attention forward through the C ABI.

    q [B, Nq, Hq, 128], k and v [B, Nk, Hkv, 128]: contiguous device tensors
    of e4m3 codes (torch.uint8 or torch.float8_e4m3fn). The function is the
    attention of the dequantized tensors (descale * codes). Allocates O
    (bf16, q's shape), LSE (float32 [B, Hq, Nq]) and the workspace with
    torch. Returns (O, LSE).
    """
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype not in (torch.uint8, torch.float8_e4m3fn):
            raise TypeError(f"{name} must hold e4m3 codes (uint8 or float8_e4m3fn)")
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("wants q [B,Nq,Hq,d], k/v [B,Nk,Hkv,d]")
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    if k.shape[0] != B or k.shape[3] != d:
        raise ValueError("q and k disagree on B or d")
    if d != 128:
        raise ValueError(f"the fp8 forward takes d=128, got d={d}")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
    if k.device != q.device or v.device != q.device:
        raise ValueError("q, k and v must be on one device")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    nbytes = fa_fwd_fp8_workspace_bytes(B, Hkv, Nk)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    st = _lib.fa_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                         B, Hq, Hkv, Nq, Nk, d, float(scale), float(q_descale), float(k_descale),
                         float(v_descale), int(bool(causal)), ws.data_ptr(), nbytes, stream)
    if st != FA_OK:
        raise FaError(st, fa_last_error())
    return out, lse


def fa_check_cu_seqlens(cu_seqlens_host, B, max_seqlen) -> int:
    """C ``fa_check_cu_seqlens``: ``cu_seqlens_host`` is an integer HOST
    address of int32 [B + 1] (or 0 / None)."""
    return _lib.fa_check_cu_seqlens(cu_seqlens_host, B, max_seqlen)


def fa_status_string(status: int) -> str:
    return _lib.fa_status_string(status).decode()


def fa_last_error() -> str:
    return _lib.fa_last_error().decode()


def fa_version() -> int:
    return _lib.fa_version()


def _check_outputs(q, out, lse, lse_shape):
    """Caller-supplied output buffers must be exactly what the kernels write:
    ``out`` like q (shape, dtype, contiguous), ``lse`` float32 of
    ``lse_shape``, contiguous. Devices are compared with q's afterwards."""
    import torch
    if out is not None:
        if tuple(out.shape) != tuple(q.shape) or out.dtype != q.dtype:
            raise ValueError(f"out must match q: shape {tuple(q.shape)}, dtype {q.dtype}; got "
                             f"{tuple(out.shape)}, {out.dtype}")
        if not out.is_contiguous():
            raise ValueError("out must be contiguous")
    if lse is not None:
        if tuple(lse.shape) != tuple(lse_shape) or lse.dtype != torch.float32:
            raise ValueError(f"lse must be float32 of shape {tuple(lse_shape)}; got "
                             f"{tuple(lse.shape)}, {lse.dtype}")
        if not lse.is_contiguous():
            raise ValueError("lse must be contiguous")


def attention_fwd(q, k, v, *, causal: bool = False, scale=None, cu_seqlens=None,
                  max_seqlen=None, out=None, lse=None, stream=None, window=None, bias=None):
    """Attention forward on torch device tensors through the C ABI.

    Fixed length: q [B, Nq, Hq, d], k and v [B, Nk, Hkv, d].
    Packed: q [T, Hq, d], k and v [T, Hkv, d], ``cu_seqlens`` int32 [nseq+1]
    on the device and ``max_seqlen`` the longest sequence (a host int).
    bf16 tensors go to ``fa_fwd``, float32 tensors to ``fa_fwd_fp32``;
    ``window`` = (left, right) selects ``fa_fwd_window`` (bf16 only);
    ``bias`` (bf16 [B or 1, Hq or 1, >= Nq, >= Nk], packed: per sequence,
    local indices) selects ``fa_fwd_bias``.
    Returns (O, LSE); O has q's shape and dtype, LSE is float32 [B, Hq, Nq]
    (packed: [Hq, T]).
    """
    import torch

    if q.dtype != k.dtype or q.dtype != v.dtype:
        raise TypeError("q, k, v must share one dtype")
    if q.dtype == torch.bfloat16:
        fn = _lib.fa_fwd
    elif q.dtype == torch.float32:
        fn = _lib.fa_fwd_fp32
    else:
        raise TypeError(f"unsupported dtype {q.dtype}; use bfloat16 or float32")
    if cu_seqlens is None:
        if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
            raise ValueError("fixed length wants q [B,Nq,Hq,d], k/v [B,Nk,Hkv,d]")
        B, Nq, Hq, d = q.shape
        Nk, Hkv = k.shape[1], k.shape[2]
        if k.shape[0] != B or k.shape[3] != d:
            raise ValueError("q and k disagree on B or d")
        lse_shape = (B, Hq, Nq)
        cu_ptr = None
    else:
        if q.dim() != 3 or k.dim() != 3 or v.shape != k.shape:
            raise ValueError("packed wants q [T,Hq,d], k/v [T,Hkv,d]")
        if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1:
            raise ValueError("cu_seqlens must be a 1-D int32 device tensor")
        if max_seqlen is None:
            raise ValueError("packed input needs max_seqlen (host int)")
        T, Hq, d = q.shape
        Hkv = k.shape[1]
        if k.shape[0] != T or k.shape[2] != d:
            raise ValueError("q and k disagree on T or d")
        B = cu_seqlens.numel() - 1
        Nq = Nk = int(max_seqlen)
        lse_shape = (Hq, T)
        cu_ptr = cu_seqlens.data_ptr()
    _check_outputs(q, out, lse, lse_shape)
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    for name, t in (("q", q), ("k", k), ("v", v), ("cu_seqlens", cu_seqlens), ("out", out),
                    ("lse", lse)):
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if t.device != q.device:
            raise ValueError(f"{name} is on {t.device}, q on {q.device}")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(lse_shape, dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    if bias is not None:
        if q.dtype != torch.bfloat16:
            raise TypeError("a bias needs bfloat16 tensors")
        if window is not None:
            raise ValueError("a window and a bias do not combine; write the window into the bias")
        sb, sh, sr = bias_strides(bias, B, Hq, Nq, Nk)
        st = _lib.fa_fwd_bias(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                              lse.data_ptr(), B, Hq, Hkv, Nq, Nk, d, float(scale),
                              int(bool(causal)), bias.data_ptr(), sb, sh, sr, cu_ptr, stream)
    elif window is not None:
        if q.dtype != torch.bfloat16:
            raise TypeError("a sliding window needs bfloat16 tensors")
        st = _lib.fa_fwd_window(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                lse.data_ptr(), B, Hq, Hkv, Nq, Nk, d, float(scale),
                                int(bool(causal)), int(window[0]), int(window[1]), cu_ptr, stream)
    else:
        st = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                B, Hq, Hkv, Nq, Nk, d, float(scale), int(bool(causal)), cu_ptr, stream)
    if st != FA_OK:
        raise FaError(st, fa_last_error())
    return out, lse


def fa_bwd_window(q, k, v, o, do, lse, dq, dk, dv, dsum, B, Hq, Hkv, Nq, Nk, d, scale, causal,
                  window_left, window_right, cu_seqlens, stream) -> int:
    """C ``fa_bwd_window``: pointers are integer device addresses (or 0 / None)."""
    return _lib.fa_bwd_window(q, k, v, o, do, lse, dq, dk, dv, dsum, B, Hq, Hkv, Nq, Nk, d, scale,
                              int(causal), window_left, window_right, cu_seqlens, stream)


def fa_bwd_bias(q, k, v, o, do, lse, dq, dk, dv, dsum, B, Hq, Hkv, Nq, Nk, d, scale, causal,
                bias, bias_stride_b, bias_stride_h, bias_stride_row, cu_seqlens, stream) -> int:
    """C ``fa_bwd_bias``: pointers are integer device addresses (or 0 / None)."""
    return _lib.fa_bwd_bias(q, k, v, o, do, lse, dq, dk, dv, dsum, B, Hq, Hkv, Nq, Nk, d, scale,
                            int(causal), bias, bias_stride_b, bias_stride_h, bias_stride_row,
                            cu_seqlens, stream)


def attention_bwd(q, k, v, o, lse, do, *, causal: bool = False, scale=None, cu_seqlens=None,
                  max_seqlen=None, stream=None, window=None, bias=None):
    """Gradients (dQ, dK, dV) of attention through the C ABI (bf16 only).

    Tensors as ``attention_fwd`` takes and returns them (``o`` and ``lse``
    from the forward call on the same inputs, with the same ``window`` or
    ``bias``), ``do`` shaped like ``o``. Allocates dQ, dK, dV and the
    float32 Dsum scratch with torch.
    """
    import torch

    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        if t.dtype != torch.bfloat16:
            raise TypeError(f"{name} must be bfloat16")
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    if lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 tensor")
    if o.shape != q.shape or do.shape != q.shape:
        raise ValueError("o and do must have q's shape")
    if cu_seqlens is None:
        if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
            raise ValueError("fixed length wants q [B,Nq,Hq,d], k/v [B,Nk,Hkv,d]")
        B, Nq, Hq, d = q.shape
        Nk, Hkv = k.shape[1], k.shape[2]
        cu_ptr = None
    else:
        if max_seqlen is None:
            raise ValueError("packed input needs max_seqlen (host int)")
        T, Hq, d = q.shape
        Hkv = k.shape[1]
        B = cu_seqlens.numel() - 1
        Nq = Nk = int(max_seqlen)
        cu_ptr = cu_seqlens.data_ptr()
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    dsum = torch.empty_like(lse)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    if bias is not None:
        if window is not None:
            raise ValueError("a window and a bias do not combine; write the window into the bias")
        sb, sh, sr = bias_strides(bias, B, Hq, Nq, Nk)
        st = _lib.fa_bwd_bias(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                              do.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                              dv.data_ptr(), dsum.data_ptr(), B, Hq, Hkv, Nq, Nk, d, float(scale),
                              int(bool(causal)), bias.data_ptr(), sb, sh, sr, cu_ptr, stream)
    elif window is not None:
        st = _lib.fa_bwd_window(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                do.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                dv.data_ptr(), dsum.data_ptr(), B, Hq, Hkv, Nq, Nk, d, float(scale),
                                int(bool(causal)), int(window[0]), int(window[1]), cu_ptr, stream)
    else:
        st = _lib.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                         lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                         dsum.data_ptr(), B, Hq, Hkv, Nq, Nk, d, float(scale), int(bool(causal)),
                         cu_ptr, stream)
    if st != FA_OK:
        raise FaError(st, fa_last_error())
    return dq, dk, dv


def attention_fwd_splitkv(q, k, v, *, num_splits: int, causal: bool = False, scale=None,
                          seqlens_k=None, stream=None):
    """Split-K/V forward (decode shapes) through the C ABI, bf16.

    q [B, Nq, Hq, d], k and v [B, Nk, Hkv, d]; ``seqlens_k`` an optional
    int32 device tensor [B] of valid keys per entry. Allocates O, LSE and the
    workspace with torch. Returns (O, LSE [B, Hq, Nq]).
    """
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != torch.bfloat16:
            raise TypeError(f"{name} must be bfloat16")
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("wants q [B,Nq,Hq,d], k/v [B,Nk,Hkv,d]")
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    if seqlens_k is not None and (seqlens_k.dtype != torch.int32 or not seqlens_k.is_cuda):
        raise ValueError("seqlens_k must be an int32 device tensor")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    nbytes = fa_fwd_splitkv_workspace_bytes(B, Hq, Nq, d, num_splits)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    st = _lib.fa_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                             lse.data_ptr(), B, Hq, Hkv, Nq, Nk, d, float(scale),
                             int(bool(causal)),
                             seqlens_k.data_ptr() if seqlens_k is not None else None,
                             int(num_splits), ws.data_ptr(), nbytes, stream)
    if st != FA_OK:
        raise FaError(st, fa_last_error())
    return o, lse
