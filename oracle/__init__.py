"""Python face of the double-precision attention oracle (``fa_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the smoke check and by the benchmark's
CPU-baseline leg.  The GPU library and its binding never import this package.

Arrays may be numpy arrays or torch tensors of any float dtype; they are widened to float32
(exact for bf16/f16/f32 storage) and the C code computes in double.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fa_oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")


class _Problem(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("mask", ctypes.c_void_p),
        ("total_lengths", ctypes.c_void_p),
        ("past_lengths", ctypes.c_void_p),
        ("batch", ctypes.c_int64),
        ("heads", ctypes.c_int64),
        ("kv_heads", ctypes.c_int64),
        ("sq", ctypes.c_int64),
        ("sk", ctypes.c_int64),
        ("kv_capacity", ctypes.c_int64),
        ("dim", ctypes.c_int64),
        ("causal", ctypes.c_int64),
        ("mask_planes", ctypes.c_int64),
        ("local_window", ctypes.c_int64),
        ("scale", ctypes.c_double),
        ("softcap", ctypes.c_double),
    ]


def build(src: str = _SRC, out: str = LIB_PATH) -> str:
    """Compile the oracle with gcc into a shared library (always recompiles)."""
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _as_f32(x) -> np.ndarray:
    if x is None:
        return None
    try:
        import torch

        if isinstance(x, torch.Tensor):
            return np.ascontiguousarray(x.detach().to("cpu", torch.float32).numpy())
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def _as_i32(x) -> Optional[np.ndarray]:
    if x is None:
        return None
    try:
        import torch

        if isinstance(x, torch.Tensor):
            return np.ascontiguousarray(x.detach().to("cpu", torch.int32).numpy())
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


class Oracle:
    """A loaded oracle library (the committed one, or a test-built variant)."""

    def __init__(self, path: str = LIB_PATH):
        self.path = path
        lib = ctypes.CDLL(path)
        lib.fa_oracle_forward.argtypes = [
            ctypes.POINTER(_Problem), ctypes.c_void_p, ctypes.c_int64, ctypes.c_int]
        lib.fa_oracle_forward.restype = ctypes.c_int
        lib.fa_oracle_rows.argtypes = [
            ctypes.POINTER(_Problem), ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
            ctypes.c_int]
        lib.fa_oracle_rows.restype = ctypes.c_int
        lib.fa_oracle_default_threads.argtypes = []
        lib.fa_oracle_default_threads.restype = ctypes.c_int
        self._lib = lib

    def default_threads(self) -> int:
        return int(self._lib.fa_oracle_default_threads())

    def _problem(self, q, k, v, sk, mask, total_lengths, past_lengths, causal, local_window,
                 scale, softcap):
        qa, ka, va = _as_f32(q), _as_f32(k), _as_f32(v)
        if qa.ndim != 4 or ka.ndim != 4 or va.shape != ka.shape:
            raise ValueError("q must be [B,H,Sq,D]; k and v [B,Hkv,C,D]")
        B, H, Sq, D = qa.shape
        Hkv, C = ka.shape[1], ka.shape[2]
        sk = C if sk is None else int(sk)
        ma = _as_f32(mask)
        planes = 0
        if ma is not None:
            if ma.ndim != 3 or ma.shape[1:] != (Sq, sk):
                raise ValueError("mask must be [planes, Sq, Sk]")
            planes = ma.shape[0]
        ta, pa = _as_i32(total_lengths), _as_i32(past_lengths)
        if scale is None:
            scale = 1.0 / np.sqrt(D)
        keep = (qa, ka, va, ma, ta, pa)
        ptr = lambda a: None if a is None else a.ctypes.data
        prob = _Problem(
            ptr(qa), ptr(ka), ptr(va), ptr(ma), ptr(ta), ptr(pa),
            B, H, Hkv, Sq, sk, C, D, 1 if causal else 0, planes, int(local_window),
            float(scale), float(softcap))
        return prob, keep, (B, H, Sq, D)

    def forward(self, q, k, v, *, sk=None, mask=None, total_lengths=None, past_lengths=None,
                causal=False, local_window=0, scale=None, softcap=0.0, out_layout="head",
                threads: int = 0) -> np.ndarray:
        """Full output in float64: [B,H,Sq,D] (head) or [B,Sq,H*D] (token)."""
        prob, keep, (B, H, Sq, D) = self._problem(
            q, k, v, sk, mask, total_lengths, past_lengths, causal, local_window, scale, softcap)
        layout = {"head": 0, "token": 1}[out_layout]
        out = np.empty((B, H, Sq, D) if layout == 0 else (B, Sq, H * D), dtype=np.float64)
        rc = self._lib.fa_oracle_forward(ctypes.byref(prob), out.ctypes.data, layout, threads)
        del keep
        if rc != 0:
            raise ValueError(f"oracle rejected the problem (status {rc})")
        return out

    def rows(self, q, k, v, rows: Sequence[Sequence[int]], *, sk=None, mask=None,
             total_lengths=None, past_lengths=None, causal=False, local_window=0, scale=None,
             softcap=0.0, threads: int = 0, **_ignored) -> np.ndarray:
        """Selected output rows (b, h, i) in float64, shape [len(rows), D]."""
        prob, keep, (B, H, Sq, D) = self._problem(
            q, k, v, sk, mask, total_lengths, past_lengths, causal, local_window, scale, softcap)
        idx = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 3))
        out = np.empty((idx.shape[0], D), dtype=np.float64)
        rc = self._lib.fa_oracle_rows(ctypes.byref(prob), idx.ctypes.data, idx.shape[0],
                                      out.ctypes.data, threads)
        del keep
        if rc != 0:
            raise ValueError(f"oracle rejected the problem (status {rc})")
        return out


_DEFAULT: Optional[Oracle] = None


def default() -> Oracle:
    """The committed oracle, compiled on first use if no build is present."""
    global _DEFAULT
    if _DEFAULT is None:
        if not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(_SRC):
            build()
        _DEFAULT = Oracle(LIB_PATH)
    return _DEFAULT


def forward(*args, **kwargs) -> np.ndarray:
    return default().forward(*args, **kwargs)


def rows(*args, **kwargs) -> np.ndarray:
    return default().rows(*args, **kwargs)
