"""Pins of the index-selection oracle (oracle/dsa_oracle.c) to values fixed independently of it:

* hand-worked cases of tests/golden/dsa_cases.json (rounding order, un-fused products, ReLU and
  weighting, canonical NaN, the allow rule, ties, padding), each citing the page passage;
* exact rational arithmetic on small integer inputs, where every float32 operation is exact;
* a brute-force selection (repeatedly take the best remaining position) on those exact scores;
* float64 scores within the float32 rounding bound on random inputs.
"""

import json
import math
import os
import struct
from fractions import Fraction

import numpy as np
import pytest

from oracle import dsa

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "dsa_cases.json")


def _num(x):
    if isinstance(x, str):
        return {"inf": math.inf, "-inf": -math.inf, "nan": math.nan}[x]
    return x


def _arr(x, dtype=np.float32):
    return np.vectorize(_num, otypes=[np.float64])(np.array(x, dtype=object)).astype(dtype)


def _cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["name"])
def test_golden_case(case):
    q, k, w, b = (_arr(case[n]) for n in ("query", "key", "weights", "bias"))
    sc, al = dsa.scores(q, k, w, b, scale=case["scale"], weights_scale=case["weights_scale"])
    if "allowed" in case:
        assert np.array_equal(al, np.array(case["allowed"], dtype=np.uint8))
    if "scores" in case:
        want = _arr(case["scores"])
        allowed = al.astype(bool)
        got = sc[allowed]
        exp = want[allowed]
        for g, e in zip(got.tolist(), exp.tolist()):
            if math.isnan(e):
                # the canonical quiet NaN, sign bit clear
                assert struct.pack("<f", g) == struct.pack("<I", 0x7FC00000), hex(struct.unpack("<I", struct.pack("<f", g))[0])
            else:
                assert g == e, (g, e)
    idx = dsa.select(sc, al, case["top_k"])
    assert np.array_equal(idx, np.array(case["indices"], dtype=np.int64)), idx


def test_minus_inf_case_with_two_slots():
    case = {c["name"]: c for c in _cases()}["minus_inf_score_is_allowed_and_lowest"]
    q, k, w, b = (_arr(case[n]) for n in ("query", "key", "weights", "bias"))
    out = dsa.index_select(q, k, w, b, top_k=2, scale=1.0)
    assert out.tolist() == [[[[0, 1]]]]


def _exact_scores(q, k, w, b, scale, wscale):
    """Scores as exact rationals (None where not allowed); valid when float32 is exact."""
    B, S, H, D = q.shape
    T = k.shape[1]
    res = {}
    for bb in range(B):
        for s in range(S):
            for t in range(T):
                bias = float(b[bb, 0, s, t])
                if not bias > -1e30:
                    res[(bb, s, t)] = None
                    continue
                total = Fraction(0)
                for h in range(H):
                    dot = sum(Fraction(float(q[bb, s, h, d])) * Fraction(float(k[bb, t, d])) for d in range(D))
                    scaled = Fraction(scale) * dot
                    total += max(scaled, Fraction(0)) * Fraction(float(w[bb, s, h])) * Fraction(wscale)
                res[(bb, s, t)] = total + Fraction(bias)
    return res


def _brute_select(values, top_k):
    """values: list of (score or None); picks the best remaining (score, then lower position)
    one at a time, then sorts the picks."""
    left = {t: v for t, v in enumerate(values) if v is not None}
    picks = []
    while left and len(picks) < top_k:
        best = min(left, key=lambda t: (-left[t], t))
        picks.append(best)
        del left[best]
    picks.sort()
    return picks + [-1] * (top_k - len(picks))


@pytest.mark.parametrize("seed", range(6))
def test_exact_small_integers(seed):
    rng = np.random.Generator(np.random.PCG64(500 + seed))
    B, S, H, D, T = 2, 3, 3, 4, 9
    q = rng.integers(-3, 4, size=(B, S, H, D)).astype(np.float32)
    k = rng.integers(-3, 4, size=(B, T, D)).astype(np.float32)
    w = rng.integers(-2, 3, size=(B, S, H)).astype(np.float32)
    b = rng.integers(-4, 5, size=(B, 1, S, T)).astype(np.float32)
    b[rng.random(size=b.shape) < 0.2] = -np.inf
    scale, wscale = 0.5, 0.25
    sc, al = dsa.scores(q, k, w, b, scale=scale, weights_scale=wscale)
    exact = _exact_scores(q, k, w, b, scale, wscale)
    for (bb, s, t), v in exact.items():
        if v is None:
            assert al[bb, s, t] == 0
        else:
            assert al[bb, s, t] == 1 and Fraction(float(sc[bb, s, t])) == v, (bb, s, t)
    for top_k in (1, 4, 9, 12):
        out = dsa.select(sc, al, top_k)
        for bb in range(B):
            for s in range(S):
                want = _brute_select([exact[(bb, s, t)] for t in range(T)], top_k)
                assert out[bb, 0, s].tolist() == want, (top_k, bb, s)


def test_float64_within_rounding_bound():
    rng = np.random.Generator(np.random.PCG64(77))
    B, S, H, D, T = 1, 2, 8, 64, 50
    q = rng.standard_normal((B, S, H, D)).astype(np.float32)
    k = rng.standard_normal((B, T, D)).astype(np.float32)
    w = rng.standard_normal((B, S, H)).astype(np.float32)
    b = rng.standard_normal((B, 1, S, T)).astype(np.float32)
    scale = 1 / 8
    sc, al = dsa.scores(q, k, w, b, scale=scale)
    assert al.all()
    dots = np.einsum("bshd,btd->bsht", q.astype(np.float64), k.astype(np.float64))
    terms = np.maximum(scale * dots, 0) * w.astype(np.float64)[..., None]
    ref = terms.sum(axis=2) + b[:, 0].astype(np.float64)
    absdots = np.einsum("bshd,btd->bsht", np.abs(q).astype(np.float64), np.abs(k).astype(np.float64))
    mag = (scale * absdots * np.abs(w).astype(np.float64)[..., None]).sum(axis=2) + np.abs(ref)
    bound = (D + H + 4) * 2.0 ** -24 * mag
    assert np.all(np.abs(sc.astype(np.float64) - ref) <= bound)
