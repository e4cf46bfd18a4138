"""MI355X (gfx950) tiled online-softmax attention forward.

Python binding of ``libfa.so`` (C ABI in ``include/fa.h``).  It only marshals arguments:
torch tensors supply device memory and the current HIP stream, and every step of the
computation runs in the library's HIP kernels.  There is no fallback: if the library or a GPU
is missing, calls raise.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

__all__ = [
    "flash_attn_fwd", "flash_attn_fwd_splitkv", "flash_attn_fwd_splitkv_noalloc",
    "splitkv_workspace_bytes", "splitkv_suggested_splits", "SPLITKV_NOALLOC_SCRATCH_BYTES",
    "check_args", "last_error", "version", "FaError", "library_path",
    "FA_OK", "FA_ERR_INVALID_ARGUMENT", "FA_ERR_UNSUPPORTED", "FA_ERR_OVERFLOW", "FA_ERR_HIP",
    "FA_DTYPE_F32", "FA_DTYPE_F16", "FA_DTYPE_BF16",
]

FA_OK = 0
FA_ERR_INVALID_ARGUMENT = -1
FA_ERR_UNSUPPORTED = -2
FA_ERR_OVERFLOW = -3
FA_ERR_HIP = -4

FA_DTYPE_F32 = 0
FA_DTYPE_F16 = 1
FA_DTYPE_BF16 = 2

# the static device scratch of flash_attn_fwd_splitkv_noalloc (FA_SPLITKV_NOALLOC_SCRATCH_BYTES)
SPLITKV_NOALLOC_SCRATCH_BYTES = 16 << 20

_DTYPE_CODE = {torch.float32: FA_DTYPE_F32, torch.float16: FA_DTYPE_F16,
               torch.bfloat16: FA_DTYPE_BF16}
_LAYOUT_CODE = {"head": 0, "token": 1}

_PKG = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_PKG, "libfa.so")

_lib = None

_ARGS = [
    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,  # q k v mask
    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,                   # total past out
    ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
    ctypes.c_int,                                                         # B H Hkv Sq Sk C D
    ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.c_float,
    ctypes.c_int, ctypes.c_int, ctypes.c_int,
]


class FaError(RuntimeError):
    """A non-OK status from libfa.so, with the library's message."""

    def __init__(self, status: int, message: str):
        super().__init__(f"flash_attn_fwd failed with status {status}: {message}")
        self.status = status
        self.message = message


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            from . import _build

            _build.build()
        lib = ctypes.CDLL(library_path)
        lib.flash_attn_fwd.argtypes = _ARGS + [ctypes.c_void_p]
        lib.flash_attn_fwd.restype = ctypes.c_int
        lib.flash_attn_fwd_splitkv.argtypes = _ARGS + [ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t,
                                                       ctypes.c_void_p]
        lib.flash_attn_fwd_splitkv.restype = ctypes.c_int
        lib.flash_attn_fwd_splitkv_noalloc.argtypes = _ARGS + [ctypes.c_int, ctypes.c_void_p]
        lib.flash_attn_fwd_splitkv_noalloc.restype = ctypes.c_int
        lib.fa_splitkv_workspace_bytes.argtypes = [ctypes.c_int] * 4
        lib.fa_splitkv_workspace_bytes.restype = ctypes.c_size_t
        lib.fa_splitkv_suggested_splits.argtypes = [ctypes.c_int] * 3
        lib.fa_splitkv_suggested_splits.restype = ctypes.c_int
        lib.fa_check_args.argtypes = list(_ARGS)
        lib.fa_check_args.restype = ctypes.c_int
        vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        dsa_args = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, f, i, vp, ctypes.c_size_t]
        lib.dsa_index_select.argtypes = dsa_args + [vp]
        lib.dsa_index_select.restype = ctypes.c_int
        lib.dsa_check_args.argtypes = dsa_args
        lib.dsa_check_args.restype = ctypes.c_int
        lib.dsa_index_select_workspace_bytes.argtypes = [i, i, i]
        lib.dsa_index_select_workspace_bytes.restype = ctypes.c_size_t
        lib.fa_last_error.argtypes = []
        lib.fa_last_error.restype = ctypes.c_char_p
        lib.fa_version.argtypes = []
        lib.fa_version.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def last_error() -> str:
    return _load().fa_last_error().decode()


def version() -> str:
    return _load().fa_version().decode()


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def check_args(*, q=None, k=None, v=None, mask=None, total_lengths=None, past_lengths=None,
               out=None, batch, heads, kv_heads, sq, sk, kv_capacity, dim, causal=0,
               mask_planes=0, local_window=0, scale=1.0, softcap=0.0, dtype=FA_DTYPE_BF16,
               mask_dtype=FA_DTYPE_F32, out_layout=0) -> int:
    """The library's validation status for raw arguments (pointers are ints or None)."""
    return _load().fa_check_args(q, k, v, mask, total_lengths, past_lengths, out, batch, heads,
                                 kv_heads, sq, sk, kv_capacity, dim, causal, mask_planes,
                                 local_window, scale, softcap, dtype, mask_dtype, out_layout)


def flash_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, sk: Optional[int] = None,
                   mask: Optional[torch.Tensor] = None,
                   total_lengths: Optional[torch.Tensor] = None,
                   past_lengths: Optional[torch.Tensor] = None, causal: bool = False,
                   local_window: int = 0, scale: Optional[float] = None, softcap: float = 0.0,
                   out_layout: str = "head", out: Optional[torch.Tensor] = None,
                   stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """Attention forward on the GPU.

    q [B,H,Sq,D]; k, v [B,Hkv,C,D] (C = kv capacity, ``sk`` <= C keys used, default C);
    mask [planes,Sq,Sk] (fp32 or q's dtype); total/past lengths int32 [B] on the device.
    Returns out [B,H,Sq,D] (``out_layout="head"``) or [B,Sq,H*D] (``"token"``).
    """
    args, out, stream, made = _marshal(q, k, v, sk, mask, total_lengths, past_lengths, causal,
                                       local_window, scale, softcap, out_layout, out, stream)
    lib = _load()
    status = lib.flash_attn_fwd(*args, stream.cuda_stream)
    if status != FA_OK:
        raise FaError(status, lib.fa_last_error().decode())
    _keep_until_done(stream, *made)
    return out


def splitkv_workspace_bytes(batch: int, kv_heads: int, dim: int, num_splits: int) -> int:
    """Workspace bytes flash_attn_fwd_splitkv needs for num_splits key spans."""
    return int(_load().fa_splitkv_workspace_bytes(batch, kv_heads, dim, num_splits))


def splitkv_suggested_splits(batch: int, kv_heads: int, sk: int) -> int:
    """A span count that fills the current device (a multiple of 4)."""
    return int(_load().fa_splitkv_suggested_splits(batch, kv_heads, sk))


def flash_attn_fwd_splitkv(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *,
                           sk: Optional[int] = None, mask: Optional[torch.Tensor] = None,
                           total_lengths: Optional[torch.Tensor] = None,
                           past_lengths: Optional[torch.Tensor] = None, causal: bool = False,
                           local_window: int = 0, scale: Optional[float] = None,
                           softcap: float = 0.0, out_layout: str = "head",
                           out: Optional[torch.Tensor] = None, num_splits: Optional[int] = None,
                           workspace: Optional[torch.Tensor] = None,
                           stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """The same attention forward with the keys split over workgroups (decode: few query rows).

    Takes bf16/f16 inputs with head dim 64 or 128 and (H / Hkv) * Sq <= 32; the mask as for
    flash_attn_fwd.
    ``workspace`` (any dtype, contiguous, on q's device) needs splitkv_workspace_bytes(...) bytes;
    it is allocated here when None.
    """
    args, out, stream, made = _marshal(q, k, v, sk, mask, total_lengths, past_lengths, causal,
                                       local_window, scale, softcap, out_layout, out, stream)
    B, _, _, D = q.shape
    Hkv, C = k.shape[1], k.shape[2]
    if num_splits is None:
        num_splits = splitkv_suggested_splits(B, Hkv, C if sk is None else int(sk))
    need = splitkv_workspace_bytes(B, Hkv, D, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
        made = made + (workspace,)
    elif not workspace.is_cuda or not workspace.is_contiguous() or workspace.device != q.device:
        raise ValueError("workspace must be a contiguous tensor on q's device")
    lib = _load()
    status = lib.flash_attn_fwd_splitkv(*args, int(num_splits), workspace.data_ptr(),
                                        workspace.numel() * workspace.element_size(), stream.cuda_stream)
    if status != FA_OK:
        raise FaError(status, lib.fa_last_error().decode())
    _keep_until_done(stream, *made)
    return out


def flash_attn_fwd_splitkv_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *,
                                   sk: Optional[int] = None, mask: Optional[torch.Tensor] = None,
                                   total_lengths: Optional[torch.Tensor] = None,
                                   past_lengths: Optional[torch.Tensor] = None,
                                   causal: bool = False, local_window: int = 0,
                                   scale: Optional[float] = None, softcap: float = 0.0,
                                   out_layout: str = "head", out: Optional[torch.Tensor] = None,
                                   num_splits: Optional[int] = None,
                                   stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """flash_attn_fwd_splitkv without a workspace: the library keeps the spans' partial states in
    a static device scratch of SPLITKV_NOALLOC_SCRATCH_BYTES (the C entry point allocates
    nothing).  Calls that overlap in time on one device race on that scratch.  Pass ``out`` to
    keep this call free of allocations on the Python side too."""
    args, out, stream, made = _marshal(q, k, v, sk, mask, total_lengths, past_lengths, causal,
                                       local_window, scale, softcap, out_layout, out, stream)
    B, _, _, _ = q.shape
    Hkv, C = k.shape[1], k.shape[2]
    if num_splits is None:
        num_splits = splitkv_suggested_splits(B, Hkv, C if sk is None else int(sk))
    lib = _load()
    status = lib.flash_attn_fwd_splitkv_noalloc(*args, int(num_splits), stream.cuda_stream)
    if status != FA_OK:
        raise FaError(status, lib.fa_last_error().decode())
    _keep_until_done(stream, *made)
    return out


def dsa_workspace_bytes(batch: int, q_seq: int, key_seq: int) -> int:
    """Workspace bytes dsa_index_select needs."""
    return int(_load().dsa_index_select_workspace_bytes(batch, q_seq, key_seq))


def dsa_check_args(query, key, weights, bias, out, batch, q_seq, heads, head_dim, key_seq, top_k,
                   scale, weights_scale, dtype, workspace, workspace_bytes) -> int:
    """The C validation of dsa_index_select on raw integer addresses (no GPU needed)."""
    return _load().dsa_check_args(query, key, weights, bias, out, batch, q_seq, heads, head_dim,
                                  key_seq, top_k, scale, weights_scale, dtype, workspace,
                                  workspace_bytes)


def dsa_index_select(query: torch.Tensor, key: torch.Tensor, weights: torch.Tensor,
                     bias: torch.Tensor, *, top_k: int, scale: float, weights_scale: float = 1.0,
                     out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                     stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """Sparse index selection: int64 [B, 1, S, top_k] positions per query row.

    query [B, S, H, D], key [B, T, D], weights [B, S, H] (one float dtype), bias [B, 1, S, T]
    float32.  ``workspace`` (contiguous, on the same device, dsa_workspace_bytes(B, S, T) bytes)
    is allocated here when None.
    """
    if query.dim() != 4 or key.dim() != 3 or weights.dim() != 3 or bias.dim() != 4:
        raise ValueError("query [B,S,H,D], key [B,T,D], weights [B,S,H], bias [B,1,S,T]")
    B, S, H, D = query.shape
    T = key.shape[1]
    if tuple(key.shape) != (B, T, D) or tuple(weights.shape) != (B, S, H) or tuple(bias.shape) != (B, 1, S, T):
        raise ValueError(f"shapes q{tuple(query.shape)} k{tuple(key.shape)} w{tuple(weights.shape)} "
                         f"bias{tuple(bias.shape)} do not match")
    if query.dtype not in _DTYPE_CODE or key.dtype != query.dtype or weights.dtype != query.dtype:
        raise ValueError("query, key and weights must share one dtype among float32, float16, bfloat16")
    if bias.dtype != torch.float32:
        raise ValueError("bias must be float32")
    made = ()
    if out is None:
        out = torch.empty((B, 1, S, int(top_k)), dtype=torch.int64, device=query.device)
        made = (out,)
    elif out.dtype != torch.int64 or tuple(out.shape) != (B, 1, S, int(top_k)):
        raise ValueError(f"out must be int64 [B, 1, S, top_k], got {out.dtype} {tuple(out.shape)}")
    for t in (query, key, weights, bias, out):
        if not t.is_cuda or not t.is_contiguous() or t.device != query.device:
            raise ValueError("every tensor must be contiguous on query's GPU")
    need = dsa_workspace_bytes(B, S, T)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=query.device)
        made = made + (workspace,)
    elif not workspace.is_cuda or not workspace.is_contiguous() or workspace.device != query.device:
        raise ValueError("workspace must be a contiguous tensor on query's device")
    if stream is None:
        stream = torch.cuda.current_stream(query.device)
    lib = _load()
    status = lib.dsa_index_select(query.data_ptr(), key.data_ptr(), weights.data_ptr(),
                                  bias.data_ptr(), out.data_ptr(), B, S, H, D, T, int(top_k),
                                  float(scale), float(weights_scale), _DTYPE_CODE[query.dtype],
                                  workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                  stream.cuda_stream)
    if status != FA_OK:
        raise FaError(status, lib.fa_last_error().decode())
    _keep_until_done(stream, *made)
    return out


def _keep_until_done(stream, *tensors) -> None:
    """Tensors allocated here come from torch's caching allocator on the current stream, while
    the kernels run on ``stream``.  Recording ``stream`` on them keeps the allocator from handing
    their memory to other work before the kernels enqueued there have finished (the caller may
    drop the workspace at once, or the output before synchronising)."""
    for t in tensors:
        t.record_stream(stream)


def _marshal(q, k, v, sk, mask, total_lengths, past_lengths, causal, local_window, scale,
             softcap, out_layout, out, stream):
    """Checks the tensors; returns the C argument list (without the stream), out, the stream and
    the tuple of tensors allocated here."""
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q must be [B,H,Sq,D]; k and v [B,Hkv,C,D]")
    B, H, Sq, D = q.shape
    Hkv, C = k.shape[1], k.shape[2]
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != D:
        raise ValueError(f"k/v shapes {tuple(k.shape)}/{tuple(v.shape)} do not match q {tuple(q.shape)}")
    if q.dtype not in _DTYPE_CODE or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share one dtype among float32, float16, bfloat16")
    tensors = [q, k, v, mask, total_lengths, past_lengths, out]
    for t in tensors:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("every tensor must live on the GPU")
            if not t.is_contiguous():
                raise ValueError("every tensor must be contiguous")
            if t.device != q.device:
                raise ValueError("every tensor must live on q's device")
    sk = C if sk is None else int(sk)
    planes = 0
    mask_dtype = FA_DTYPE_F32
    if mask is not None:
        if mask.dim() != 3 or mask.shape[1] != Sq or mask.shape[2] != sk:
            raise ValueError(f"mask must be [planes, Sq={Sq}, Sk={sk}], got {tuple(mask.shape)}")
        if mask.dtype not in _DTYPE_CODE:
            raise ValueError("mask must be float32 or q's dtype")
        planes = mask.shape[0]
        mask_dtype = _DTYPE_CODE[mask.dtype]
    for name, t in (("total_lengths", total_lengths), ("past_lengths", past_lengths)):
        if t is not None and (t.dtype != torch.int32 or t.shape != (B,)):
            raise ValueError(f"{name} must be int32 [B]")
    layout = _LAYOUT_CODE[out_layout]
    made = ()
    if out is None:
        shape = (B, H, Sq, D) if layout == 0 else (B, Sq, H * D)
        out = torch.empty(shape, dtype=q.dtype, device=q.device)
        made = (out,)
    elif out.dtype != q.dtype or out.numel() != B * H * Sq * D:
        raise ValueError("out must match q's dtype and element count")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    args = [_ptr(q), _ptr(k), _ptr(v), _ptr(mask), _ptr(total_lengths), _ptr(past_lengths), _ptr(out),
            B, H, Hkv, Sq, sk, C, D, 1 if causal else 0, planes, int(local_window), float(scale),
            float(softcap), _DTYPE_CODE[q.dtype], mask_dtype, layout]
    return args, out, stream, made
