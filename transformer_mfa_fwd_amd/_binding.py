"""ctypes binding of libmfa (include/mfa.h).

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, their device pointers and torch's current HIP stream are passed to
the C ABI, and a non-zero status raises MFAError.  Every step of the attention
forward runs in the library's HIP kernels; there is no fallback.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmfa.so")

MFA_F32, MFA_F16, MFA_BF16 = 0, 1, 2
PATH_AUTO, PATH_GENERIC, PATH_MFMA, PATH_SPLIT_DECODE = 0, 1, 2, 3
PATH_NAMES = {PATH_AUTO: "auto", PATH_GENERIC: "generic", PATH_MFMA: "mfma",
              PATH_SPLIT_DECODE: "split_decode"}
_DTYPE_CODES = {torch.float32: MFA_F32, torch.float16: MFA_F16, torch.bfloat16: MFA_BF16}

EXPORTED = ("mfa_fwd", "mfa_fwd_workspace_size", "mfa_fwd_ws", "mfa_fwd_ex", "mfa_fwd_plan",
            "mfa_decode_len", "mfa_decode_len_workspace_size", "mfa_decode_len_noalloc", "mfa_decode_masked",
            "mfa_decode_masked_workspace_size", "mfa_packed_qkv_fwd",
            "mfa_varlen_fwd", "mfa_varlen_workspace_size", "mfa_fwd_bias_dropout",
            "mfa_bwd", "mfa_bwd_workspace_size",
            "mfa_status_string", "mfa_last_error", "mfa_version", "mfa_set_kernel_events")


class MFAError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


_lib = None

_I = ctypes.c_int
_P = ctypes.c_void_p
_F = ctypes.c_float
_FWD_ARGS = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _I, _I, _F, _P, _I]


def load_library(path: str = LIB_PATH):
    """Load libmfa.so (built in-tree by transformer_mfa_fwd_amd/build.py)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"libmfa.so not found at {path}; build it with "
                          "`python transformer_mfa_fwd_amd/build.py`")
    lib = ctypes.CDLL(path)
    lib.mfa_fwd.restype = _I
    lib.mfa_fwd.argtypes = _FWD_ARGS + [_P]
    lib.mfa_fwd_ws.restype = _I
    lib.mfa_fwd_ws.argtypes = _FWD_ARGS + [_P, ctypes.c_size_t, _P]
    lib.mfa_fwd_ex.restype = _I
    lib.mfa_fwd_ex.argtypes = _FWD_ARGS + [_I, _I, _P, ctypes.c_size_t, _P]
    lib.mfa_fwd_workspace_size.restype = ctypes.c_size_t
    lib.mfa_fwd_workspace_size.argtypes = [_I] * 7
    lib.mfa_fwd_plan.restype = _I
    lib.mfa_fwd_plan.argtypes = [_I] * 7 + [ctypes.POINTER(_I)]
    lib.mfa_decode_len.restype = _I
    lib.mfa_decode_len.argtypes = [_P] * 6 + [_I] * 6 + [_F, _F, _I, _I, _P, ctypes.c_size_t, _P]
    lib.mfa_decode_masked.restype = _I
    lib.mfa_decode_len_noalloc.restype = _I
    lib.mfa_decode_len_noalloc.argtypes = [_P] * 6 + [_I] * 6 + [_F, _F, _I, _I, _P]
    lib.mfa_decode_masked.argtypes = [_P] * 6 + [_I] * 5 + [_F, _I, _F, _I, _I, _P, ctypes.c_size_t, _P]
    lib.mfa_decode_masked_workspace_size.restype = ctypes.c_size_t
    lib.mfa_decode_masked_workspace_size.argtypes = [_I] * 7
    lib.mfa_fwd_bias_dropout.restype = _I
    lib.mfa_fwd_bias_dropout.argtypes = _FWD_ARGS[:-1] + [_P, _I, _I, _I, _I, _F, ctypes.c_ulonglong, _I, _P]
    lib.mfa_bwd.restype = _I
    lib.mfa_bwd.argtypes = [_P] * 9 + [_I] * 6 + [_F, _I, _I, _I, _F, _P, _P, _I, _I, _I, _I, _F,
                                                  ctypes.c_ulonglong, _I, _P, ctypes.c_size_t, _P]
    lib.mfa_bwd_workspace_size.restype = ctypes.c_size_t
    lib.mfa_bwd_workspace_size.argtypes = [_I] * 3
    lib.mfa_varlen_fwd.restype = _I
    lib.mfa_varlen_fwd.argtypes = [_P] * 7 + [_I] * 6 + [_F, _I, _I, _F, _I, _P, ctypes.c_size_t, _P]
    lib.mfa_varlen_workspace_size.restype = ctypes.c_size_t
    lib.mfa_varlen_workspace_size.argtypes = [_I] * 5
    lib.mfa_packed_qkv_fwd.restype = _I
    lib.mfa_packed_qkv_fwd.argtypes = [_P] * 4 + [_I] * 3 + [_F, _I, _F, _I, _P]
    lib.mfa_decode_len_workspace_size.restype = ctypes.c_size_t
    lib.mfa_decode_len_workspace_size.argtypes = [_I] * 8
    lib.mfa_status_string.restype = ctypes.c_char_p
    lib.mfa_status_string.argtypes = [_I]
    lib.mfa_last_error.restype = ctypes.c_char_p
    lib.mfa_last_error.argtypes = []
    lib.mfa_version.restype = _I
    lib.mfa_version.argtypes = []
    lib.mfa_set_kernel_events.restype = None
    lib.mfa_set_kernel_events.argtypes = [_P, _P]
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        lib = load_library()
        raise MFAError(status, f"libmfa: {lib.mfa_status_string(status).decode()}: "
                               f"{lib.mfa_last_error().decode()}")


def _dims(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor):
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q must be [B, Lq, Hq, D]; k and v [B, Lk, Hkv, D]")
    B, Lq, Hq, D = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != D:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)}")
    return B, Lq, k.shape[1], Hq, k.shape[2], D


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, causal: bool = False,
        window: int = 0, q_offset: Optional[int] = None, softcap: float = 0.0,
        key_mask: Optional[torch.Tensor] = None, scale: Optional[float] = None,
        out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
        return_lse: bool = True, path: int = PATH_AUTO, splits: int = 0,
        workspace: Optional[torch.Tensor] = None, bias: Optional[torch.Tensor] = None,
        dropout_p: float = 0.0, seed: int = 0, stream=None
        ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Attention forward through libmfa.

    q [B, Lq, Hq, D]; k, v [B, Lk, Hkv, D] (same dtype, contiguous, on one
    GPU); key_mask [B, Lk] float32 or None.  q_offset defaults to Lk - Lq and
    scale to 1/sqrt(D).  Returns (out [B, Lq, Hq, D], lse [B, Hq, Lq] float32
    or None).  ``path``/``splits`` force a kernel path (mfa_fwd_ex);
    ``workspace`` is a caller-owned uint8 device tensor (mfa_fwd_ws).
    ``bias`` (a contiguous float32 GPU tensor [bB, bH, bLq, bLk], each 1 or
    B, Hq, Lq, Lk) and ``dropout_p``/``seed`` select mfa_fwd_bias_dropout.
    """
    lib = load_library()
    B, Lq, Lk, Hq, Hkv, D = _dims(q, k, v)
    if q.dtype not in _DTYPE_CODES or k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError(f"dtypes must match and be one of float32/float16/bfloat16 "
                        f"(got {q.dtype}, {k.dtype}, {v.dtype})")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    if key_mask is not None:
        if key_mask.dtype != torch.float32 or tuple(key_mask.shape) != (B, Lk) or \
                not key_mask.is_cuda or not key_mask.is_contiguous():
            raise ValueError("key_mask must be a contiguous float32 GPU tensor of shape [B, Lk]")
    if q_offset is None:
        q_offset = Lk - Lq
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be contiguous and match q")
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=q.device)
    elif lse is not None and (lse.shape != (B, Hq, Lq) or lse.dtype != torch.float32):
        raise ValueError("lse must be float32 [B, Hq, Lq]")
    args = [_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Lq, Lk, Hq, Hkv, D,
            float(scale), int(bool(causal)), int(window), int(q_offset), float(softcap),
            _ptr(key_mask), _DTYPE_CODES[q.dtype]]
    if bias is not None or dropout_p > 0.0:
        if path != PATH_AUTO or splits or workspace is not None:
            raise ValueError("bias and dropout take neither a forced path nor a workspace")
        dims = [1, 1, 1, 1]
        if bias is not None:
            if bias.dim() != 4 or bias.dtype != torch.float32 or not bias.is_cuda or \
                    not bias.is_contiguous():
                raise ValueError("bias must be a contiguous float32 GPU tensor [bB, bH, bLq, bLk]")
            dims = [int(x) for x in bias.shape]
        with torch.cuda.device(q.device):
            _check(lib.mfa_fwd_bias_dropout(*args[:-1], _ptr(bias), *dims, float(dropout_p),
                                            ctypes.c_ulonglong(int(seed) & (2 ** 64 - 1)), args[-1],
                                            _stream(stream)))
        return out, lse
    with torch.cuda.device(q.device):
        s = _stream(stream)
        ws_ptr = _ptr(workspace)
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        if path != PATH_AUTO or splits:
            _check(lib.mfa_fwd_ex(*args, int(path), int(splits), ws_ptr, ws_bytes, s))
        elif workspace is not None:
            _check(lib.mfa_fwd_ws(*args, ws_ptr, ws_bytes, s))
        else:
            _check(lib.mfa_fwd(*args, s))
    return out, lse


def _decode_len_dims(q, k_cache, v_cache, d_len):
    B, R, Lmax, Hq, Hkv, D = _dims(q, k_cache, v_cache)
    if q.dtype not in (torch.float16, torch.bfloat16) or k_cache.dtype != q.dtype or \
            v_cache.dtype != q.dtype:
        raise TypeError(f"dtypes must match and be float16 or bfloat16 "
                        f"(got {q.dtype}, {k_cache.dtype}, {v_cache.dtype})")
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    if d_len.dtype != torch.int32 or tuple(d_len.shape) != (B,) or not d_len.is_cuda or \
            not d_len.is_contiguous():
        raise ValueError("d_len must be a contiguous int32 GPU tensor of shape [B]")
    return B, R, Lmax, Hq, Hkv, D


def decode_len(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
               d_len: torch.Tensor, *, softcap: float = 0.0, scale: Optional[float] = None,
               out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
               return_lse: bool = True, splits: int = 0,
               workspace: Optional[torch.Tensor] = None, stream=None
               ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Decode over the first d_len[b] rows of a fixed-capacity cache
    (mfa_decode_len).

    q [B, R, Hq, D]; k_cache, v_cache [B, Lmax, Hkv, D] (fp16 or bf16, one
    dtype, contiguous, on one GPU); d_len int32 [B] on the same GPU, read by
    the kernels when they run.  Row r of batch b attends to keys
    0 .. d_len[b] - R + r.  Returns (out [B, R, Hq, D], lse [B, Hq, R] float32
    or None).  ``workspace`` (a uint8 device tensor of at least
    decode_len_workspace_size bytes) makes the call allocation-free, as graph
    capture needs.
    """
    lib = load_library()
    B, R, Lmax, Hq, Hkv, D = _decode_len_dims(q, k_cache, v_cache, d_len)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be contiguous and match q")
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, R), dtype=torch.float32, device=q.device)
    elif lse is not None and (lse.shape != (B, Hq, R) or lse.dtype != torch.float32):
        raise ValueError("lse must be float32 [B, Hq, R]")
    with torch.cuda.device(q.device):
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        _check(lib.mfa_decode_len(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(lse),
                                  _ptr(d_len), B, R, Lmax, Hq, Hkv, D, float(scale), float(softcap),
                                  _DTYPE_CODES[q.dtype], int(splits), _ptr(workspace), ws_bytes,
                                  _stream(stream)))
    return out, lse


def decode_len_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                       d_len: torch.Tensor, out: torch.Tensor, lse: Optional[torch.Tensor] = None, *,
                       softcap: float = 0.0, scale: Optional[float] = None, splits: int = 0,
                       stream=None) -> None:
    """decode_len into caller-given out [B, R, Hq, D] (and lse [B, Hq, R]
    float32, or None) with the split partials in the library's static device
    scratch (mfa_decode_len_noalloc): neither this function nor the library
    allocates device memory.  Calls whose kernels overlap on one device share
    that scratch and race."""
    lib = load_library()
    B, R, Lmax, Hq, Hkv, D = _decode_len_dims(q, k_cache, v_cache, d_len)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous() or out.device != q.device:
        raise ValueError("out must be contiguous and match q")
    if lse is not None and (lse.shape != (B, Hq, R) or lse.dtype != torch.float32 or
                            not lse.is_contiguous() or lse.device != q.device):
        raise ValueError("lse must be contiguous float32 [B, Hq, R] on q's device")
    with torch.cuda.device(q.device):
        _check(lib.mfa_decode_len_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(lse),
                                          _ptr(d_len), B, R, Lmax, Hq, Hkv, D, float(scale), float(softcap),
                                          _DTYPE_CODES[q.dtype], int(splits), _stream(stream)))


def decode_masked(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                  d_mask: torch.Tensor, *, window: int = 0, softcap: float = 0.0,
                  scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                  lse: Optional[torch.Tensor] = None, return_lse: bool = True, splits: int = 0,
                  workspace: Optional[torch.Tensor] = None, stream=None
                  ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Single-query decode over a fixed-capacity cache whose valid keys are
    marked by a device key mask (mfa_decode_masked).

    q [B, 1, Hq, D]; k_cache, v_cache [B, Lmax, Hkv, D] (fp16 or bf16, one
    dtype, contiguous, on one GPU); d_mask float32 [B, Lmax] on the same GPU,
    read by the kernels when they run.  The query sits at each batch's last
    valid key; ``window`` > 0 keeps only the valid keys after that position
    minus the window.  Returns (out [B, 1, Hq, D], lse [B, Hq, 1] float32 or
    None).  ``workspace`` (a uint8 device tensor of at least
    decode_masked_workspace_size bytes) makes the call allocation-free, as
    graph capture needs.
    """
    lib = load_library()
    B, R, Lmax, Hq, Hkv, D = _dims(q, k_cache, v_cache)
    if R != 1:
        raise ValueError("q must hold one query row per batch: [B, 1, Hq, D]")
    if q.dtype not in (torch.float16, torch.bfloat16) or k_cache.dtype != q.dtype or \
            v_cache.dtype != q.dtype:
        raise TypeError(f"dtypes must match and be float16 or bfloat16 "
                        f"(got {q.dtype}, {k_cache.dtype}, {v_cache.dtype})")
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    if d_mask.dtype != torch.float32 or tuple(d_mask.shape) != (B, Lmax) or not d_mask.is_cuda or \
            not d_mask.is_contiguous():
        raise ValueError("d_mask must be a contiguous float32 GPU tensor of shape [B, Lmax]")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be contiguous and match q")
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, 1), dtype=torch.float32, device=q.device)
    elif lse is not None and (lse.shape != (B, Hq, 1) or lse.dtype != torch.float32):
        raise ValueError("lse must be float32 [B, Hq, 1]")
    with torch.cuda.device(q.device):
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        _check(lib.mfa_decode_masked(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(lse),
                                     _ptr(d_mask), B, Lmax, Hq, Hkv, D, float(scale), int(window),
                                     float(softcap), _DTYPE_CODES[q.dtype], int(splits), _ptr(workspace),
                                     ws_bytes, _stream(stream)))
    return out, lse


def packed_qkv_fwd(qkv: torch.Tensor, seq_bounds: torch.Tensor, num_heads: int, *,
                   window: int = 0, softcap: float = 0.0, scale: Optional[float] = None,
                   out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                   return_lse: bool = True, stream=None
                   ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Bidirectional attention over sequences packed back to back in one fused
    QKV tensor (mfa_packed_qkv_fwd).

    qkv [L, 3 * num_heads * D] (per row: query heads, key heads, value heads;
    fp32, fp16 or bf16, contiguous, on a GPU); seq_bounds int32 [L, 2] on the
    same GPU, row r's sequence being rows [seq_bounds[r, 0], seq_bounds[r, 1]).
    Returns (out [L, num_heads * D], lse [num_heads, L] float32 or None).
    """
    lib = load_library()
    if qkv.dim() != 2 or qkv.shape[1] % (3 * num_heads) != 0:
        raise ValueError("qkv must be [L, 3 * num_heads * head_dim]")
    L = qkv.shape[0]
    H = int(num_heads)
    D = qkv.shape[1] // (3 * H)
    if qkv.dtype not in _DTYPE_CODES:
        raise TypeError(f"qkv dtype must be float32, float16 or bfloat16 (got {qkv.dtype})")
    if not qkv.is_cuda or not qkv.is_contiguous():
        raise ValueError("qkv must be a contiguous GPU tensor")
    if seq_bounds.dtype != torch.int32 or tuple(seq_bounds.shape) != (L, 2) or \
            not seq_bounds.is_cuda or not seq_bounds.is_contiguous():
        raise ValueError("seq_bounds must be a contiguous int32 GPU tensor of shape [L, 2]")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((L, H * D), dtype=qkv.dtype, device=qkv.device)
    elif tuple(out.shape) != (L, H * D) or out.dtype != qkv.dtype or not out.is_contiguous():
        raise ValueError("out must be contiguous [L, num_heads * head_dim] in qkv's dtype")
    if lse is None and return_lse:
        lse = torch.empty((H, L), dtype=torch.float32, device=qkv.device)
    elif lse is not None and (tuple(lse.shape) != (H, L) or lse.dtype != torch.float32):
        raise ValueError("lse must be float32 [num_heads, L]")
    with torch.cuda.device(qkv.device):
        _check(lib.mfa_packed_qkv_fwd(_ptr(qkv), _ptr(seq_bounds), _ptr(out), _ptr(lse), L, H, D,
                                      float(scale), int(window), float(softcap),
                                      _DTYPE_CODES[qkv.dtype], _stream(stream)))
    return out, lse


def varlen_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens_q: torch.Tensor,
               cu_seqlens_k: torch.Tensor, *, causal: bool = False, window: int = 0,
               softcap: float = 0.0, scale: Optional[float] = None,
               out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
               return_lse: bool = True, workspace: Optional[torch.Tensor] = None, stream=None
               ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Attention over sequences packed with separate query and key packings
    (mfa_varlen_fwd).

    q [total_q, Hq, D]; k, v [total_k, Hkv, D] (one dtype, contiguous, on one
    GPU); cu_seqlens_q / cu_seqlens_k int32 [batch + 1] prefix sums on the same
    GPU.  Returns (out [total_q, Hq, D], lse [Hq, total_q] float32 or None).
    """
    lib = load_library()
    if q.dim() != 3 or k.dim() != 3 or k.shape != v.shape or k.shape[2] != q.shape[2]:
        raise ValueError("q must be [total_q, Hq, D]; k and v [total_k, Hkv, D]")
    Tq, Hq, D = q.shape
    Tk, Hkv = k.shape[0], k.shape[1]
    if q.dtype not in _DTYPE_CODES or k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError(f"dtypes must match and be one of float32/float16/bfloat16 "
                        f"(got {q.dtype}, {k.dtype}, {v.dtype})")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    batch = cu_seqlens_q.numel() - 1
    for name, t in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        if t.dtype != torch.int32 or t.dim() != 1 or t.numel() != batch + 1 or not t.is_cuda or \
                not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous int32 GPU tensor of batch + 1 entries")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be contiguous and match q")
    if lse is None and return_lse:
        lse = torch.empty((Hq, Tq), dtype=torch.float32, device=q.device)
    elif lse is not None and (tuple(lse.shape) != (Hq, Tq) or lse.dtype != torch.float32):
        raise ValueError("lse must be float32 [Hq, total_q]")
    with torch.cuda.device(q.device):
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        _check(lib.mfa_varlen_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(cu_seqlens_q),
                                  _ptr(cu_seqlens_k), batch, Tq, Tk, Hq, Hkv, D, float(scale),
                                  int(bool(causal)), int(window), float(softcap), _DTYPE_CODES[q.dtype],
                                  _ptr(workspace), ws_bytes, _stream(stream)))
    return out, lse


def bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor, dout: torch.Tensor,
        lse: torch.Tensor, *, causal: bool = False, window: int = 0, q_offset: Optional[int] = None,
        softcap: float = 0.0, key_mask: Optional[torch.Tensor] = None, scale: Optional[float] = None,
        bias: Optional[torch.Tensor] = None, dropout_p: float = 0.0, seed: int = 0,
        dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
        dv: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None, stream=None):
    """Gradients (dq, dk, dv) of the forward for the output gradient dout
    (mfa_bwd).  out and lse are the forward's results; every option must
    repeat the forward call's."""
    lib = load_library()
    B, Lq, Lk, Hq, Hkv, D = _dims(q, k, v)
    if q.dtype not in _DTYPE_CODES or k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one of float32/float16/bfloat16")
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    if out.shape != q.shape or dout.shape != q.shape or out.dtype != q.dtype or dout.dtype != q.dtype:
        raise ValueError("out and dout must match q")
    if lse.shape != (B, Hq, Lq) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be contiguous float32 [B, Hq, Lq]")
    if key_mask is not None and (key_mask.dtype != torch.float32 or tuple(key_mask.shape) != (B, Lk)):
        raise ValueError("key_mask must be float32 [B, Lk]")
    dims = [1, 1, 1, 1]
    if bias is not None:
        if bias.dim() != 4 or bias.dtype != torch.float32 or not bias.is_contiguous():
            raise ValueError("bias must be a contiguous float32 tensor [bB, bH, bLq, bLk]")
        dims = [int(x) for x in bias.shape]
    if q_offset is None:
        q_offset = Lk - Lq
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if t.shape != ref.shape or t.dtype != ref.dtype or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous and match its input")
    with torch.cuda.device(q.device):
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        _check(lib.mfa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk),
                           _ptr(dv), B, Lq, Lk, Hq, Hkv, D, float(scale), int(bool(causal)), int(window),
                           int(q_offset), float(softcap), _ptr(key_mask), _ptr(bias), *dims, float(dropout_p),
                           ctypes.c_ulonglong(int(seed) & (2 ** 64 - 1)), _DTYPE_CODES[q.dtype],
                           _ptr(workspace), ws_bytes, _stream(stream)))
    return dq, dk, dv


def bwd_workspace_size(B: int, Lq: int, Hq: int) -> int:
    return int(load_library().mfa_bwd_workspace_size(B, Lq, Hq))


def varlen_workspace_size(total_q: int, total_k: int, Hkv: int, D: int, dtype: torch.dtype) -> int:
    return int(load_library().mfa_varlen_workspace_size(int(total_q), int(total_k), int(Hkv), int(D),
                                                        _DTYPE_CODES[dtype]))


def decode_len_workspace_size(B, R, Lmax, Hq, Hkv, D, dtype: torch.dtype, splits: int = 0) -> int:
    return int(load_library().mfa_decode_len_workspace_size(B, R, Lmax, Hq, Hkv, D,
                                                            _DTYPE_CODES[dtype], int(splits)))


def decode_masked_workspace_size(B, Lmax, Hq, Hkv, D, dtype: torch.dtype, splits: int = 0) -> int:
    return int(load_library().mfa_decode_masked_workspace_size(B, Lmax, Hq, Hkv, D, _DTYPE_CODES[dtype],
                                                               int(splits)))


def workspace_size(B, Lq, Lk, Hq, Hkv, D, dtype: torch.dtype) -> int:
    return int(load_library().mfa_fwd_workspace_size(B, Lq, Lk, Hq, Hkv, D, _DTYPE_CODES[dtype]))


def plan(B, Lq, Lk, Hq, Hkv, D, dtype: torch.dtype):
    """(path name, split count) that mfa_fwd would use."""
    s = ctypes.c_int(0)
    p = load_library().mfa_fwd_plan(B, Lq, Lk, Hq, Hkv, D, _DTYPE_CODES[dtype], ctypes.byref(s))
    return PATH_NAMES.get(p, str(p)), s.value


def version() -> int:
    return int(load_library().mfa_version())


def set_kernel_events(begin=None, end=None):
    """Events (torch.cuda.Event, already recorded once so that they exist, or
    None) that later calls on this thread record around their main kernel
    (mfa_set_kernel_events)."""
    def handle(e):
        return None if e is None else ctypes.c_void_p(e.cuda_event)
    load_library().mfa_set_kernel_events(handle(begin), handle(end))
