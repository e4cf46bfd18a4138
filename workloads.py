"""Seeded synthetic attention inputs, shared by the GPU path's tests/benchmark and by the oracle.

This module only draws numbers and arranges them into tensors. It holds none of the
attention arithmetic (no scores, no masking rule, no softmax): both sides of a parity
check receive exactly the same stored values from here and compute on their own.

Recipe (the same for every workload):
  * ``numpy.random.Generator(PCG64(seed))``; draw order is q, k, v, then lengths, then mask.
  * q/k/v are ``standard_normal(float32)`` values; 16-bit workloads round them to bf16/f16
    by round-to-nearest-even through ``torch.Tensor.to``.  The device and the oracle consume
    the same rounded values.
  * KV-cache prefill: ``past[b] ~ U{0..max_past}`` (inclusive), ``total = past + Sq``;
    K/V rows at or beyond ``min(total[b], Sk)`` are filled with NaN, so a kernel that reads and
    uses them cannot match.
  * Key-rule edges: ``past`` and ``total`` drawn independently (``total`` up to the capacity, so
    it can fall short of ``past + Sq`` or pass ``Sk``), or given explicitly (zero and negative
    values included).
  * Masked workload: an fp32 additive mask ``[B, Sq, Sk]`` with i.i.d. Bernoulli(p) entries set
    to ``-inf`` (else ``0.0``), plus a few seeded query rows per batch set entirely to ``-inf``.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

_TORCH_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass
class Problem:
    """One attention forward problem: host tensors plus the op's scalar arguments."""

    name: str
    q: torch.Tensor  # [B, H, Sq, D]
    k: torch.Tensor  # [B, Hkv, C, D]
    v: torch.Tensor  # [B, Hkv, C, D]
    sk: int
    causal: bool = False
    local_window: int = 0
    scale: float = 1.0
    softcap: float = 0.0
    mask: Optional[torch.Tensor] = None  # [planes, Sq, Sk]
    total_lengths: Optional[torch.Tensor] = None  # int32 [B]
    past_lengths: Optional[torch.Tensor] = None  # int32 [B]
    out_layout: str = "head"  # "head" -> [B,H,Sq,D]; "token" -> [B,Sq,H*D]

    @property
    def batch(self) -> int:
        return self.q.shape[0]

    @property
    def heads(self) -> int:
        return self.q.shape[1]

    @property
    def kv_heads(self) -> int:
        return self.k.shape[1]

    @property
    def sq(self) -> int:
        return self.q.shape[2]

    @property
    def dim(self) -> int:
        return self.q.shape[3]

    @property
    def kv_capacity(self) -> int:
        return self.k.shape[2]

    @property
    def dtype(self) -> str:
        return {v: k for k, v in _TORCH_DTYPES.items()}[self.q.dtype]

    def kwargs(self) -> dict:
        """Keyword arguments shared by the GPU binding and the oracle wrapper."""
        return dict(
            sk=self.sk,
            mask=self.mask,
            total_lengths=self.total_lengths,
            past_lengths=self.past_lengths,
            causal=self.causal,
            local_window=self.local_window,
            scale=self.scale,
            softcap=self.softcap,
            out_layout=self.out_layout,
        )

    def to(self, device) -> "Problem":
        """A copy with every tensor moved to ``device``."""
        moved = {}
        for f in dataclasses.fields(self):
            val = getattr(self, f.name)
            moved[f.name] = val.to(device) if isinstance(val, torch.Tensor) else val
        return Problem(**moved)


def _normal(rng: np.random.Generator, shape, dtype: str, amp: float = 1.0,
            dist: str = "normal") -> torch.Tensor:
    if dist == "normal":
        x = rng.standard_normal(size=shape, dtype=np.float32)
    elif dist == "neg_uniform":
        # one-signed values in [-1, 0), the range of the prior-art parity test's generator
        x = -rng.random(size=shape, dtype=np.float32)
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    if amp != 1.0:
        x = x * np.float32(amp)
    return torch.from_numpy(x).to(_TORCH_DTYPES[dtype])


def make_problem(
    *,
    name: str = "custom",
    seed: int,
    batch: int,
    heads: int,
    kv_heads: int,
    sq: int,
    sk: int,
    dim: int,
    dtype: str,
    kv_capacity: Optional[int] = None,
    causal: bool = False,
    local_window: int = 0,
    scale: Optional[float] = None,
    softcap: float = 0.0,
    amp: float = 1.0,
    dist: str = "normal",
    lengths: Optional[str] = None,
    max_past: int = 0,
    max_total: Optional[int] = None,
    total_values=None,
    past_values=None,
    nan_beyond_total: bool = False,
    key_ramp: float = 0.0,
    mask: Optional[str] = None,
    mask_planes: Optional[int] = None,
    mask_dtype: str = "f32",
    mask_p: float = 0.1,
    mask_ramp: float = 0.0,
    mask_offset: float = 0.0,
    q_scale: float = 1.0,
    dead_rows: int = 0,
    out_layout: str = "head",
) -> Problem:
    """Draw one problem.

    ``lengths``: ``None`` (no length tensors), ``"past"`` (past ~ U{0..max_past}, total = past + sq),
    ``"total"`` (only total_lengths ~ U{0..sk}), ``"past_only"`` (only past_lengths),
    ``"indep"`` (past ~ U{0..max_past} and, drawn after it, total ~ U{0..max_total}, max_total
    defaulting to the capacity) or ``"explicit"`` (``total_values`` / ``past_values``, either
    may be None; no numbers are drawn).
    ``nan_beyond_total``: K/V rows at or past ``min(total[b], sk)`` become NaN.
    ``key_ramp``: ``key_ramp * j`` is added to every element of key row j before rounding, so
    that scores drift by a large amount along the keys (rising for some query rows, falling for
    others).
    ``mask``: ``None``, ``"bernoulli"`` (-inf with probability ``mask_p``, else 0), ``"normal"``
    (finite N(0,1) values with Bernoulli -inf holes), ``"ramp"`` (``mask_ramp * j`` for key j,
    with Bernoulli -inf holes) or ``"extreme"`` (finite values at the end of the mask type's
    range, see below, with Bernoulli -inf holes); ``mask_planes`` defaults to ``batch``.
    ``mask_offset``: added (in float32) to the finite values of a ``"normal"`` or ``"ramp"`` mask.
    ``q_scale``: every element of Q is multiplied by it after the draw (0 gives all-zero scores,
    so that the scores are the mask values exactly, whatever their magnitude).
    ``dead_rows``: query rows per mask plane set entirely to -inf.
    ``dist``: ``"normal"`` (N(0,1)) or ``"neg_uniform"`` (U[-1,0)), times ``amp``.
    """
    capacity = sk if kv_capacity is None else kv_capacity
    rng = np.random.Generator(np.random.PCG64(seed))
    q = _normal(rng, (batch, heads, sq, dim), dtype, amp, dist)
    k = _normal(rng, (batch, kv_heads, capacity, dim), dtype, amp, dist)
    v = _normal(rng, (batch, kv_heads, capacity, dim), dtype, amp, dist)
    if q_scale != 1.0:
        q = (q.float() * np.float32(q_scale)).to(q.dtype)
    if key_ramp:
        ramp = torch.arange(capacity, dtype=torch.float32).view(1, 1, capacity, 1) * np.float32(key_ramp)
        k = (k.float() + ramp).to(k.dtype)

    total = past = None
    if lengths == "past":
        past_np = rng.integers(0, max_past, size=batch, endpoint=True).astype(np.int32)
        past = torch.from_numpy(past_np)
        total = torch.from_numpy((past_np + np.int32(sq)).astype(np.int32))
    elif lengths == "total":
        total = torch.from_numpy(rng.integers(0, sk, size=batch, endpoint=True).astype(np.int32))
    elif lengths == "past_only":
        past = torch.from_numpy(rng.integers(0, max_past, size=batch, endpoint=True).astype(np.int32))
    elif lengths == "indep":
        past = torch.from_numpy(rng.integers(0, max_past, size=batch, endpoint=True).astype(np.int32))
        hi = capacity if max_total is None else max_total
        total = torch.from_numpy(rng.integers(0, hi, size=batch, endpoint=True).astype(np.int32))
    elif lengths == "explicit":
        if total_values is not None:
            total = torch.tensor(list(total_values), dtype=torch.int32)
        if past_values is not None:
            past = torch.tensor(list(past_values), dtype=torch.int32)
    elif lengths is not None:
        raise ValueError(f"unknown lengths recipe {lengths!r}")

    if nan_beyond_total and total is not None:
        for b in range(batch):
            t = max(min(int(total[b]), sk), 0)
            if t < capacity:
                k[b, :, t:, :] = float("nan")
                v[b, :, t:, :] = float("nan")

    mask_t = None
    if mask is not None:
        planes = batch if mask_planes is None else mask_planes
        holes = rng.random(size=(planes, sq, sk), dtype=np.float32) < np.float32(mask_p)
        if mask == "bernoulli":
            m = np.zeros((planes, sq, sk), dtype=np.float32)
        elif mask == "normal":
            m = rng.standard_normal(size=(planes, sq, sk), dtype=np.float32)
        elif mask == "ramp":
            m = np.broadcast_to(np.arange(sk, dtype=np.float32) * np.float32(mask_ramp),
                                (planes, sq, sk)).copy()
        elif mask == "extreme":
            # finite values at the end of the mask type's range: row i % 3 == 0 holds only the
            # most negative finite value, row 1 mixes it with 0, row 2 mixes it with half of it
            big = np.float32(torch.finfo(_TORCH_DTYPES[mask_dtype]).max)
            pick = rng.random(size=(planes, sq, sk), dtype=np.float32) < np.float32(0.5)
            m = np.full((planes, sq, sk), -big, dtype=np.float32)
            m[:, 1::3, :] = np.where(pick[:, 1::3, :], np.float32(0.0), -big)
            m[:, 2::3, :] = np.where(pick[:, 2::3, :], -big / np.float32(2.0), -big)
            del pick
        else:
            raise ValueError(f"unknown mask recipe {mask!r}")
        if mask_offset and mask in ("normal", "ramp"):
            m = m + np.float32(mask_offset)
        m[holes] = -np.inf
        del holes
        if dead_rows:
            for p in range(planes):
                rows = rng.choice(sq, size=min(dead_rows, sq), replace=False)
                m[p, rows, :] = -np.inf
        mask_t = torch.from_numpy(m)
        if mask_dtype != "f32":
            mask_t = mask_t.to(_TORCH_DTYPES[mask_dtype])

    return Problem(
        name=name,
        q=q,
        k=k,
        v=v,
        sk=sk,
        causal=causal,
        local_window=local_window,
        scale=(1.0 / math.sqrt(dim)) if scale is None else scale,
        softcap=softcap,
        mask=mask_t,
        total_lengths=total,
        past_lengths=past,
        out_layout=out_layout,
    )


# The five named workloads at full size.  Seeds are the workload's ordinal (1..5).  A sixth,
# vae_decoder, exercises the wide fp32 head dim (384) of the pictor page's second build of its
# joint-attention kernel; the page gives no shape for it, so it takes a 64 x 64 latent (4096
# tokens) with four heads, non-causal, token-major output like the DiT workload.
WORKLOADS = {
    "tiny": dict(seed=1, batch=1, heads=1, kv_heads=1, sq=64, sk=64, dim=64, dtype="f32"),
    "dit_joint": dict(
        seed=2, batch=1, heads=24, kv_heads=24, sq=1536, sk=1536, dim=128, dtype="f32",
        out_layout="token",
    ),
    "gqa_causal": dict(
        seed=3, batch=4, heads=32, kv_heads=8, sq=2048, sk=2048, dim=128, dtype="bf16", causal=True,
    ),
    "kv_cache_prefill": dict(
        seed=4, batch=8, heads=32, kv_heads=8, sq=512, sk=4096, kv_capacity=4096, dim=128,
        dtype="f16", causal=True, local_window=1024, softcap=50.0, lengths="past", max_past=2048,
        nan_beyond_total=True,
    ),
    "masked_long": dict(
        seed=5, batch=2, heads=16, kv_heads=16, sq=4096, sk=4096, dim=64, dtype="bf16",
        mask="bernoulli", mask_p=0.1, dead_rows=4,
    ),
    "vae_decoder": dict(
        seed=6, batch=1, heads=4, kv_heads=4, sq=4096, sk=4096, dim=384, dtype="f32",
        out_layout="token",
    ),
    # one decode step of the GQA shape (32 query heads on 8 KV heads, head dim 128) against a
    # full 8192-row cache per sequence, 16 sequences: the split-key path's workload
    "gqa_decode": dict(
        seed=7, batch=16, heads=32, kv_heads=8, sq=1, sk=8192, dim=128, dtype="bf16", causal=True,
    ),
}

# Reduced copies with the same structure (dtype, features, GQA group, layout), small enough for
# the full oracle to finish in seconds while still spanning several tiles and a ragged tail.
SMALL_WORKLOADS = {
    "tiny": dict(WORKLOADS["tiny"]),
    "dit_joint": dict(WORKLOADS["dit_joint"], heads=3, kv_heads=3, sq=333, sk=333),
    "gqa_causal": dict(WORKLOADS["gqa_causal"], batch=2, heads=8, kv_heads=2, sq=300, sk=300),
    "kv_cache_prefill": dict(
        WORKLOADS["kv_cache_prefill"], batch=3, heads=8, kv_heads=2, sq=77, sk=640, kv_capacity=640,
        local_window=160, max_past=400,
    ),
    "masked_long": dict(WORKLOADS["masked_long"], heads=4, kv_heads=4, sq=261, sk=390),
    "vae_decoder": dict(WORKLOADS["vae_decoder"], heads=2, kv_heads=2, sq=200, sk=200),
    "gqa_decode": dict(WORKLOADS["gqa_decode"], batch=3, heads=8, kv_heads=2, sk=1000),
}

# workloads that bench.py runs through the split-key entry point
SPLITKV_WORKLOADS = {"gqa_decode"}


def workload(name: str, small: bool = False, **overrides) -> Problem:
    """The named workload (full size, or its reduced copy) with optional field overrides."""
    table = SMALL_WORKLOADS if small else WORKLOADS
    params = dict(table[name])
    params.update(overrides)
    return make_problem(name=name + ("_small" if small else ""), **params)


# ------------------------------------------------------------------------------------------
# Sparse index selection (the dsa_index_select.rs page): seeded inputs only, no arithmetic of
# the operation.

@dataclasses.dataclass
class DsaProblem:
    name: str
    query: torch.Tensor     # [B, S, H, D]
    key: torch.Tensor       # [B, T, D]
    weights: torch.Tensor   # [B, S, H]
    bias: torch.Tensor      # [B, 1, S, T] float32
    top_k: int
    scale: float
    weights_scale: float

    @property
    def dtype(self) -> str:
        return {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}[self.query.dtype]

    def to(self, device) -> "DsaProblem":
        return DsaProblem(self.name, self.query.to(device), self.key.to(device),
                          self.weights.to(device), self.bias.to(device), self.top_k, self.scale,
                          self.weights_scale)

    def kwargs(self) -> dict:
        return dict(top_k=self.top_k, scale=self.scale, weights_scale=self.weights_scale)


def make_dsa_problem(*, name: str = "dsa", seed: int, batch: int, q_seq: int, heads: int,
                     head_dim: int, key_seq: int, top_k: int, dtype: str, bias: str = "causal",
                     scale: Optional[float] = None, weights_scale: float = 1.0,
                     int_values: bool = False, hole_p: float = 0.0,
                     overflow_keys: int = 0) -> DsaProblem:
    """Draw one index-selection problem.

    Values are N(0,1) (or, with ``int_values``, integers in [-2, 2], which make ties common).
    ``bias``: ``"causal"`` (0 for positions up to the row's bottom-right causal limit
    T - S + s, beyond it alternately -inf and the float32 minimum, both below -1e30),
    ``"random"`` (N(0,1) values) or ``"zero"``; ``hole_p`` sets that fraction of positions to
    -inf.  ``overflow_keys`` key rows are scaled by 1e30 so that their products overflow.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    tdt = _TORCH_DTYPES[dtype]

    def draw(shape):
        if int_values:
            return torch.from_numpy(rng.integers(-2, 3, size=shape).astype(np.float32)).to(tdt)
        return torch.from_numpy(rng.standard_normal(size=shape, dtype=np.float32)).to(tdt)

    query = draw((batch, q_seq, heads, head_dim))
    key = draw((batch, key_seq, head_dim))
    weights = draw((batch, q_seq, heads))
    if overflow_keys and key_seq:
        rows = rng.choice(key_seq, size=min(overflow_keys, key_seq), replace=False)
        key = key.float()
        key[:, rows, :] = 3e38   # products overflow to +-inf (f16 stores inf itself)
        key = key.to(tdt)
    if bias == "causal":
        b = np.zeros((batch, 1, q_seq, key_seq), dtype=np.float32)
        fill = np.where(np.arange(key_seq) % 2 == 0, -np.inf, np.finfo(np.float32).min).astype(np.float32)
        for s in range(q_seq):
            limit = key_seq - q_seq + s
            b[:, 0, s, limit + 1:] = fill[limit + 1:]
    elif bias == "random":
        b = rng.standard_normal(size=(batch, 1, q_seq, key_seq), dtype=np.float32)
    elif bias == "zero":
        b = np.zeros((batch, 1, q_seq, key_seq), dtype=np.float32)
    else:
        raise ValueError(f"unknown bias recipe {bias!r}")
    if hole_p:
        b[rng.random(size=b.shape) < hole_p] = -np.inf
    return DsaProblem(name=name, query=query, key=key, weights=weights, bias=torch.from_numpy(b),
                      top_k=top_k, scale=(1.0 / math.sqrt(head_dim)) if scale is None else scale,
                      weights_scale=weights_scale)


# The index-selection workload: one decode step of a 64-head, 128-dim indexer over 32768 cached
# positions for 8 sequences, keeping 2048 positions per query row (the page gives no shape; these
# are the sizes such indexers are described with).  The small copy keeps the structure.
DSA_WORKLOADS = {
    "dsa_decode": dict(seed=8, batch=8, q_seq=1, heads=64, head_dim=128, key_seq=32768,
                       top_k=2048, dtype="bf16", bias="causal"),
}
SMALL_DSA_WORKLOADS = {
    "dsa_decode": dict(DSA_WORKLOADS["dsa_decode"], batch=2, heads=8, key_seq=3000, top_k=256),
}


def dsa_workload(name: str, small: bool = False, **overrides) -> DsaProblem:
    table = SMALL_DSA_WORKLOADS if small else DSA_WORKLOADS
    params = dict(table[name])
    params.update(overrides)
    return make_dsa_problem(name=name, **params)
