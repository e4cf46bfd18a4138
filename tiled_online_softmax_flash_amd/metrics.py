"""Work accounting for the attention forward: attended keys, algorithmic flops and bytes.

Host-side arithmetic on the key rule of fa.h (the `logical_sk` / `causal_max` / `local_min`
definitions of `flash_attention_body` on the onnx-runtime-ep-cuda page
`src/kernels/flash_attention.rs`).  The throughput metric counts only attended keys:
flops = 4 * D * sum over (b, h, i) of |attended keys of row i|, i.e. 2*D for Q.K^T plus 2*D
for P.V per attended score; the additive mask does not reduce the count.
"""

from __future__ import annotations

from typing import Optional

import numpy as np


def attended_counts(batch: int, sq: int, sk: int, causal: bool, local_window: int,
                    total_lengths: Optional[np.ndarray] = None,
                    past_lengths: Optional[np.ndarray] = None) -> np.ndarray:
    """int64 [batch, sq]: number of attended keys of each query row (closed form of the rule)."""
    i = np.arange(sq, dtype=np.int64)[None, :]
    L = np.full((batch, 1), sk, dtype=np.int64)
    if total_lengths is not None:
        L = np.minimum(L, np.asarray(total_lengths, dtype=np.int64).reshape(batch, 1))
    L = np.maximum(L, 0)
    if past_lengths is not None:
        cmax = np.asarray(past_lengths, dtype=np.int64).reshape(batch, 1) + i
    else:
        cmax = L - sq + i
    lo = np.maximum(0, cmax + 1 - local_window) if local_window > 0 else np.zeros_like(cmax)
    hi = np.minimum(L - 1, cmax) if causal else np.broadcast_to(L - 1, cmax.shape)
    return np.maximum(0, hi - lo + 1)


def _np(t):
    if t is None:
        return None
    try:
        import torch

        if isinstance(t, torch.Tensor):
            return t.detach().cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(t)


def problem_work(prob) -> dict:
    """Attended scores, Sk_eff, flops and algorithmic HBM bytes of a workloads.Problem."""
    counts = attended_counts(prob.batch, prob.sq, prob.sk, prob.causal, prob.local_window,
                             _np(prob.total_lengths), _np(prob.past_lengths))
    scores = int(counts.sum()) * prob.heads
    esz = prob.q.element_size()
    # bytes: Q read once, O written once, each attended K/V row of every KV head read once,
    # the mask read once per (plane, row, key) it covers.
    q_bytes = prob.q.numel() * esz
    kv_rows = 0
    for b in range(prob.batch):
        c = counts[b]
        if (c > 0).any():
            # union of attended ranges over rows: keys in [min lo, max hi]
            i = np.nonzero(c > 0)[0]
            kv_rows += _union_rows(prob, b, i)
    kv_bytes = 2 * kv_rows * prob.kv_heads * prob.dim * esz
    mask_bytes = 0 if prob.mask is None else prob.mask.numel() * prob.mask.element_size()
    return dict(
        attended_scores=scores,
        sk_eff=scores / max(1, prob.batch * prob.heads * prob.sq),
        flops=4 * prob.dim * scores,
        bytes=2 * q_bytes + kv_bytes + mask_bytes,
    )


def _union_rows(prob, b: int, rows: np.ndarray) -> int:
    total = _np(prob.total_lengths)
    past = _np(prob.past_lengths)
    L = prob.sk if total is None else min(int(total[b]), prob.sk)
    L = max(L, 0)
    first, last = int(rows.min()), int(rows.max())
    cmax_first = (int(past[b]) if past is not None else L - prob.sq) + first
    cmax_last = (int(past[b]) if past is not None else L - prob.sq) + last
    lo = max(0, cmax_first + 1 - prob.local_window) if prob.local_window > 0 else 0
    hi = min(L - 1, cmax_last) if prob.causal else L - 1
    return max(0, hi - lo + 1)
