"""Python face of the index-selection oracle (``dsa_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the smoke check and by the benchmark's
CPU-baseline leg.  The GPU library and its binding never import it.

The operation is the sparse index selection of the onnx-runtime-ep-cuda page
``src/kernels/dsa_index_select.rs`` (module documentation): head-weighted, ReLU'd, scaled dot
products of every key position, plus an f32 bias that also masks (bias <= -1e30), then the
top ``min(#allowed, top_k)`` positions by (score descending in total order, position ascending),
written in ascending position order and padded with -1.  Scores are float32 in the page's fixed
order; ``dsa_oracle.c`` states it in full.

Inputs may be numpy arrays or torch tensors; query/key/weights of any float dtype are widened to
float32 (exact for f16/bf16), the bias must hold float32 values.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dsa_oracle.c")
LIB_PATH = os.path.join(_HERE, "libdsa_oracle.so")


def build(src: str = _SRC, out: str = LIB_PATH) -> str:
    """Compile with gcc (always recompiles).  -ffp-contract=off keeps products and sums apart."""
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _f32(x) -> np.ndarray:
    try:
        import torch

        if isinstance(x, torch.Tensor):
            return np.ascontiguousarray(x.detach().to("cpu", torch.float32).numpy())
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


class DsaOracle:
    def __init__(self, path: str = LIB_PATH):
        lib = ctypes.CDLL(path)
        i64, f32, vp = ctypes.c_int64, ctypes.c_float, ctypes.c_void_p
        lib.dsa_oracle_scores.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, f32, f32, vp, vp]
        lib.dsa_oracle_scores.restype = ctypes.c_int
        lib.dsa_oracle_select.argtypes = [vp, vp, i64, i64, i64, vp]
        lib.dsa_oracle_select.restype = ctypes.c_int
        self._lib = lib

    def scores(self, query, key, weights, bias, *, scale: float, weights_scale: float = 1.0):
        """(scores float32 [B, S, T], allowed uint8 [B, S, T])."""
        q, k, w, bi = _f32(query), _f32(key), _f32(weights), _f32(bias)
        if q.ndim != 4 or k.ndim != 3 or w.ndim != 3 or bi.ndim != 4:
            raise ValueError("query [B,S,H,D], key [B,T,D], weights [B,S,H], bias [B,1,S,T]")
        B, S, H, D = q.shape
        T = k.shape[1]
        if k.shape != (B, T, D) or w.shape != (B, S, H) or bi.shape != (B, 1, S, T):
            raise ValueError(f"shape mismatch: q{q.shape} k{k.shape} w{w.shape} bias{bi.shape}")
        sc = np.empty((B, S, T), dtype=np.float32)
        al = np.empty((B, S, T), dtype=np.uint8)
        rc = self._lib.dsa_oracle_scores(q.ctypes.data, k.ctypes.data, w.ctypes.data,
                                         bi.ctypes.data, B, S, H, D, T, float(scale),
                                         float(weights_scale), sc.ctypes.data, al.ctypes.data)
        if rc != 0:
            raise RuntimeError("oracle scoring failed")
        return sc, al

    def select(self, scores, allowed, top_k: int) -> np.ndarray:
        """int64 [B, 1, S, top_k] from scores/allowed [B, S, T]."""
        sc = np.ascontiguousarray(scores, dtype=np.float32)
        al = np.ascontiguousarray(allowed, dtype=np.uint8)
        B, S, T = sc.shape
        out = np.empty((B, 1, S, int(top_k)), dtype=np.int64)
        rc = self._lib.dsa_oracle_select(sc.ctypes.data, al.ctypes.data, B * S, T, int(top_k),
                                         out.ctypes.data)
        if rc != 0:
            raise MemoryError("oracle selection ran out of memory")
        return out

    def index_select(self, query, key, weights, bias, *, top_k: int, scale: float,
                     weights_scale: float = 1.0) -> np.ndarray:
        sc, al = self.scores(query, key, weights, bias, scale=scale, weights_scale=weights_scale)
        return self.select(sc, al, top_k)


_DEFAULT: Optional[DsaOracle] = None


def default() -> DsaOracle:
    """The committed oracle, compiled on first use if no build is present.  The environment
    variable DSA_ORACLE_LIB names another build instead (the mutant tests use it)."""
    global _DEFAULT
    if _DEFAULT is None:
        other = os.environ.get("DSA_ORACLE_LIB")
        if other:
            _DEFAULT = DsaOracle(other)
            return _DEFAULT
        if not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(_SRC):
            build()
        _DEFAULT = DsaOracle(LIB_PATH)
    return _DEFAULT


def scores(*args, **kwargs):
    return default().scores(*args, **kwargs)


def select(*args, **kwargs):
    return default().select(*args, **kwargs)


def index_select(*args, **kwargs):
    return default().index_select(*args, **kwargs)
