"""The host-side work accounting (attended keys per row) against the hand-worked attended sets
and against the oracle's probability rows (CPU only)."""

import numpy as np

from oracle_pins import golden_cases
from tiled_online_softmax_flash_amd.metrics import attended_counts, problem_work
import workloads


def test_counts_match_hand_worked_sets():
    for case in golden_cases():
        counts = attended_counts(case["batch"], case["sq"], case["sk"], case["causal"],
                                 case["local_window"], case["total_lengths"], case["past_lengths"])
        for b, i, keys in case["attended"]:
            assert counts[b, i] == len(keys), (case["name"], b, i)


def test_counts_match_oracle_support(orc):
    rng = np.random.Generator(np.random.PCG64(7))
    for trial in range(20):
        B, Sq, C = 2, int(rng.integers(1, 12)), int(rng.integers(1, 14))
        sk = int(rng.integers(0, C + 1))
        causal = bool(rng.integers(0, 2))
        W = int(rng.integers(0, 5))
        total = rng.integers(-1, C + 3, size=B).astype(np.int32) if rng.integers(0, 2) else None
        past = rng.integers(0, 8, size=B).astype(np.int32) if rng.integers(0, 2) else None
        if sk == 0:
            continue
        q = rng.standard_normal((B, 1, Sq, C)).astype(np.float32)
        k = rng.standard_normal((B, 1, C, C)).astype(np.float32)
        v = np.broadcast_to(np.eye(C, dtype=np.float32), (B, 1, C, C)).copy()
        out = orc.forward(q, k, v, sk=sk, causal=causal, local_window=W, total_lengths=total,
                          past_lengths=past, scale=0.3)
        support = (out[:, 0] > 0).sum(axis=-1)
        counts = attended_counts(B, Sq, sk, causal, W, total, past)
        assert np.array_equal(support, counts), trial


def test_headline_workload_sizes():
    w = problem_work(workloads.workload("gqa_causal"))
    assert w["attended_scores"] == 4 * 32 * (2048 * 2049 // 2)
    assert abs(w["sk_eff"] - 1024.5) < 1e-9
    assert w["flops"] == 4 * 128 * w["attended_scores"]
    assert abs(w["flops"] / 1e9 - 137.51) < 0.01
