"""Pins for the double-precision oracle: facts fixed by the pages or by mathematics.

Every pin takes an ``Oracle`` object and raises ``AssertionError`` when the oracle disagrees.
They are run against the committed oracle (``test_oracle_pins.py``) and against deliberately
broken copies of it (``test_oracle_mutants.py``), where at least one pin must fail per copy.

None of these re-types the oracle's own code path: attended-key sets come from the hand-worked
fixture ``golden/attended_sets.json``; expected values come from closed forms, from a
brute-force naive softmax that takes those sets as given, from torch's float64 CPU
scaled-dot-product attention, or from invariances the definition implies.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

_GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "attended_sets.json")


def golden_cases():
    with open(_GOLDEN) as f:
        return json.load(f)["cases"]


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _randn(rng, *shape):
    return rng.standard_normal(size=shape).astype(np.float32)


def _lengths(case, key):
    val = case[key]
    return None if val is None else np.asarray(val, dtype=np.int32)


# ------------------------------------------------------------------------------------------
# closed forms


def pin_single_key_returns_v(orc):
    """One key: the softmax weight is exactly 1, so every row returns that key's V row."""
    rng = _rng(11)
    q, k, v = _randn(rng, 2, 4, 5, 7), _randn(rng, 2, 2, 1, 7), _randn(rng, 2, 2, 1, 7)
    out = orc.forward(q, k, v)
    for b in range(2):
        for h in range(4):
            for i in range(5):
                assert np.array_equal(out[b, h, i], v[b, h // 2, 0].astype(np.float64)), (b, h, i)


def pin_window_one_returns_diagonal(orc):
    """Causal with window 1 keeps only key cmax = past + i: the output is that V row exactly."""
    case = next(c for c in golden_cases() if c["name"] == "window_one")
    rng = _rng(12)
    B, Sq, C = case["batch"], case["sq"], case["kv_capacity"]
    q, k, v = _randn(rng, B, 2, Sq, 3), _randn(rng, B, 1, C, 3), _randn(rng, B, 1, C, 3)
    out = orc.forward(q, k, v, sk=case["sk"], causal=True, local_window=1,
                      total_lengths=_lengths(case, "total_lengths"),
                      past_lengths=_lengths(case, "past_lengths"))
    for b, i, keys in case["attended"]:
        (j,) = keys
        for h in range(2):
            assert np.array_equal(out[b, h, i], v[b, 0, j].astype(np.float64)), (b, h, i)


def pin_first_causal_row_is_v0(orc):
    """Square causal attention: row 0 attends key 0 only."""
    rng = _rng(13)
    q, k, v = _randn(rng, 1, 3, 10, 6), _randn(rng, 1, 3, 10, 6), _randn(rng, 1, 3, 10, 6)
    out = orc.forward(q, k, v, causal=True)
    for h in range(3):
        assert np.array_equal(out[0, h, 0], v[0, h, 0].astype(np.float64))


def pin_identical_keys_mean(orc):
    """All keys equal: every attended key gets the same weight, so rows are means of V."""
    rng = _rng(14)
    Sq = Sk = 9
    q = _randn(rng, 1, 2, Sq, 5)
    k = np.repeat(_randn(rng, 1, 1, 1, 5), Sk, axis=2)
    v = _randn(rng, 1, 1, Sk, 5)
    out = orc.forward(q, k, v, causal=True)
    for h in range(2):
        for i in range(Sq):
            want = v[0, 0, : i + 1].astype(np.float64).mean(axis=0)
            assert np.allclose(out[0, h, i], want, rtol=0, atol=1e-12), (h, i)


def pin_scale_zero_gives_mean_over_attended(orc):
    """scale = 0 makes every attended score 0: each row is the mean of its attended V rows."""
    for n, case in enumerate(golden_cases()):
        rng = _rng(100 + n)
        B, Sq, C = case["batch"], case["sq"], case["kv_capacity"]
        q, k, v = _randn(rng, B, 2, Sq, 4), _randn(rng, B, 1, C, 4), _randn(rng, B, 1, C, 4)
        out = orc.forward(q, k, v, sk=case["sk"], causal=case["causal"],
                          local_window=case["local_window"], scale=0.0,
                          total_lengths=_lengths(case, "total_lengths"),
                          past_lengths=_lengths(case, "past_lengths"))
        for b, i, keys in case["attended"]:
            for h in range(2):
                if keys:
                    want = v[b, 0, keys].astype(np.float64).mean(axis=0)
                    assert np.allclose(out[b, h, i], want, rtol=0, atol=1e-12), (case["name"], b, i)
                else:
                    assert np.array_equal(out[b, h, i], np.zeros(4)), (case["name"], b, i)


def pin_probability_rows(orc):
    """With V = identity, an output row is the probability row: non-negative, zero off the
    hand-worked attended set, summing to one (or all zero when nothing is attended)."""
    for n, case in enumerate(golden_cases()):
        rng = _rng(200 + n)
        B, Sq, C = case["batch"], case["sq"], case["kv_capacity"]
        q, k = _randn(rng, B, 3, Sq, C), _randn(rng, B, 1, C, C)
        v = np.broadcast_to(np.eye(C, dtype=np.float32), (B, 1, C, C)).copy()
        out = orc.forward(q, k, v, sk=case["sk"], causal=case["causal"],
                          local_window=case["local_window"], scale=0.5,
                          total_lengths=_lengths(case, "total_lengths"),
                          past_lengths=_lengths(case, "past_lengths"))
        for b, i, keys in case["attended"]:
            for h in range(3):
                p = out[b, h, i]
                off = np.ones(C, dtype=bool)
                off[keys] = False
                assert np.all(p >= 0), (case["name"], b, h, i)
                assert np.all(p[off] == 0.0), (case["name"], b, h, i, p)
                if keys:
                    assert abs(p.sum() - 1.0) <= 1e-12, (case["name"], b, h, i)
                    assert np.all(p[keys] > 0), (case["name"], b, h, i)
                else:
                    assert np.all(p == 0.0)


def pin_softcap_two_keys(orc):
    """Two keys, D = 1: the output is the logistic blend v0*sig(x0-x1) + v1*sig(x1-x0), with
    x_j = c*tanh(scale*q*k_j/c) + mask_j (softcap before the additive mask)."""
    scale, cap = 0.9, 2.0
    qv, kv, vv, mv = 1.7, (2.3, -1.1), (0.25, -3.0), (0.4, -0.7)
    q = np.array(qv, np.float32).reshape(1, 1, 1, 1)
    k = np.array(kv, np.float32).reshape(1, 1, 2, 1)
    v = np.array(vv, np.float32).reshape(1, 1, 2, 1)
    m = np.array(mv, np.float32).reshape(1, 1, 2)
    x = [cap * math.tanh(scale * float(np.float32(qv)) * float(np.float32(kj)) / cap) + float(np.float32(mj))
         for kj, mj in zip(kv, mv)]
    sig = lambda t: 1.0 / (1.0 + math.exp(-t))
    want = float(np.float32(vv[0])) * sig(x[0] - x[1]) + float(np.float32(vv[1])) * sig(x[1] - x[0])
    got = orc.forward(q, k, v, mask=m, scale=scale, softcap=cap)[0, 0, 0, 0]
    assert abs(got - want) <= 1e-13, (got, want)


# ------------------------------------------------------------------------------------------
# brute force and a library routine


def _naive_row(qrow, K, V, keys, scale, softcap, mrow):
    """Naive softmax (no max subtraction) in Python floats over a given key set."""
    if not keys:
        return [0.0] * V.shape[1]
    weights = []
    for j in keys:
        s = scale * math.fsum(float(a) * float(b) for a, b in zip(qrow, K[j]))
        if softcap > 0:
            s = softcap * math.tanh(s / softcap)
        if mrow is not None:
            s += float(mrow[j])
        weights.append(math.exp(s))
    tot = math.fsum(weights)
    return [math.fsum(w * float(V[j][d]) for w, j in zip(weights, keys)) / tot
            for d in range(V.shape[1])]


def pin_brute_force_naive_softmax(orc):
    """Tiny inputs, every golden case, with softcap and a finite per-batch mask: the oracle
    equals a naive exp/sum softmax over the hand-worked attended sets to 1e-12."""
    for n, case in enumerate(golden_cases()):
        rng = _rng(300 + n)
        B, Sq, C, Sk = case["batch"], case["sq"], case["kv_capacity"], case["sk"]
        H, Hkv, D = 4, 2, 3
        q, k, v = _randn(rng, B, H, Sq, D), _randn(rng, B, Hkv, C, D), _randn(rng, B, Hkv, C, D)
        mask = (0.5 * _randn(rng, B, Sq, Sk)).astype(np.float32)
        for softcap in (0.0, 1.5):
            out = orc.forward(q, k, v, sk=Sk, causal=case["causal"],
                              local_window=case["local_window"], scale=0.8, softcap=softcap,
                              mask=mask, total_lengths=_lengths(case, "total_lengths"),
                              past_lengths=_lengths(case, "past_lengths"))
            for b, i, keys in case["attended"]:
                for h in range(H):
                    kvh = h // (H // Hkv)
                    want = _naive_row(q[b, h, i], k[b, kvh], v[b, kvh], keys, 0.8, softcap,
                                      mask[b, i])
                    assert np.allclose(out[b, h, i], want, rtol=0, atol=1e-12), (
                        case["name"], softcap, b, h, i)


def pin_matches_torch_sdpa_float64(orc):
    """Where the op reduces to torch's scaled_dot_product_attention (no lengths, window or
    softcap; causal only with Sq == Sk, whose top-left and bottom-right alignments agree),
    the oracle matches torch's float64 CPU result."""
    import torch.nn.functional as F

    rng = _rng(400)
    cases = [
        dict(B=2, H=6, Hkv=3, Sq=7, Sk=11, D=5, causal=False, mask=False),
        dict(B=2, H=4, Hkv=1, Sq=9, Sk=9, D=8, causal=True, mask=False),
        dict(B=2, H=4, Hkv=4, Sq=6, Sk=13, D=4, causal=False, mask=True),
    ]
    for c in cases:
        q = _randn(rng, c["B"], c["H"], c["Sq"], c["D"])
        k = _randn(rng, c["B"], c["Hkv"], c["Sk"], c["D"])
        v = _randn(rng, c["B"], c["Hkv"], c["Sk"], c["D"])
        mask = _randn(rng, c["B"], c["Sq"], c["Sk"]) if c["mask"] else None
        out = orc.forward(q, k, v, causal=c["causal"], scale=0.37, mask=mask)
        tq, tk, tv = (torch.from_numpy(a).double() for a in (q, k, v))
        attn_mask = None if mask is None else torch.from_numpy(mask).double()[:, None]
        want = F.scaled_dot_product_attention(
            tq, tk, tv, attn_mask=attn_mask, is_causal=c["causal"], scale=0.37,
            enable_gqa=c["H"] != c["Hkv"])
        assert np.allclose(out, want.numpy(), rtol=0, atol=1e-12), c


# ------------------------------------------------------------------------------------------
# invariances of the definition


def pin_mask_row_shift_invariance(orc):
    """Adding a constant to a whole mask row (holes stay -inf) leaves the output unchanged."""
    rng = _rng(500)
    q, k, v = _randn(rng, 1, 2, 6, 4), _randn(rng, 1, 2, 8, 4), _randn(rng, 1, 2, 8, 4)
    # values on a 2^-10 grid, so that adding the shifts below is exact in float32
    mask = (np.round(_randn(rng, 1, 6, 8) * 1024) / 1024).astype(np.float32)
    mask[0, 2, 3] = -np.inf
    shift = np.array([3.5, -2.0, 7.25, 0.0, -11.0, 1.0], np.float32)[None, :, None]
    a = orc.forward(q, k, v, mask=mask)
    b = orc.forward(q, k, v, mask=mask + shift)
    assert np.allclose(a, b, rtol=0, atol=1e-12)


def pin_key_permutation_invariance(orc):
    """Non-causal, unmasked attention is a set function of the (key, value) pairs."""
    rng = _rng(501)
    q, k, v = _randn(rng, 2, 2, 5, 4), _randn(rng, 2, 2, 9, 4), _randn(rng, 2, 2, 9, 4)
    perm = rng.permutation(9)
    a = orc.forward(q, k, v)
    b = orc.forward(q, k[:, :, perm], v[:, :, perm])
    assert np.allclose(a, b, rtol=0, atol=1e-12)


def pin_gqa_equals_repeated_heads(orc):
    """Grouped heads equal plain multi-head attention on K/V repeated group-wise
    (consecutive query heads share a KV head)."""
    rng = _rng(502)
    q, k, v = _randn(rng, 2, 6, 5, 4), _randn(rng, 2, 2, 7, 4), _randn(rng, 2, 2, 7, 4)
    a = orc.forward(q, k, v, causal=True, local_window=3)
    b = orc.forward(q, np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1), causal=True,
                    local_window=3)
    assert np.allclose(a, b, rtol=0, atol=0)


def pin_wide_window_is_no_window(orc):
    """A window at least as long as the key range removes nothing."""
    rng = _rng(503)
    q, k, v = _randn(rng, 1, 2, 6, 4), _randn(rng, 1, 1, 6, 4), _randn(rng, 1, 1, 6, 4)
    for causal in (False, True):
        a = orc.forward(q, k, v, causal=causal)
        b = orc.forward(q, k, v, causal=causal, local_window=6)
        c = orc.forward(q, k, v, causal=causal, local_window=1000)
        assert np.array_equal(a, b) and np.array_equal(a, c)


def pin_huge_softcap_is_no_softcap(orc):
    rng = _rng(504)
    q, k, v = _randn(rng, 1, 2, 6, 4), _randn(rng, 1, 1, 6, 4), _randn(rng, 1, 1, 6, 4)
    a = orc.forward(q, k, v, scale=2.0)
    b = orc.forward(q, k, v, scale=2.0, softcap=1e30)
    assert np.allclose(a, b, rtol=0, atol=1e-13)


def pin_token_major_is_transpose(orc):
    rng = _rng(505)
    q, k, v = _randn(rng, 2, 3, 5, 4), _randn(rng, 2, 3, 7, 4), _randn(rng, 2, 3, 7, 4)
    head = orc.forward(q, k, v, causal=True)
    tok = orc.forward(q, k, v, causal=True, out_layout="token")
    assert tok.shape == (2, 5, 12)
    assert np.array_equal(tok, head.transpose(0, 2, 1, 3).reshape(2, 5, 12))


def pin_masked_key_equals_deleted_key(orc):
    """A -inf mask entry for key j equals deleting key j from K, V and the mask."""
    rng = _rng(506)
    q, k, v = _randn(rng, 1, 2, 4, 3), _randn(rng, 1, 2, 6, 3), _randn(rng, 1, 2, 6, 3)
    mask = _randn(rng, 1, 4, 6)
    mask[:, :, 2] = -np.inf
    a = orc.forward(q, k, v, mask=mask)
    keep = [0, 1, 3, 4, 5]
    b = orc.forward(q, k[:, :, keep], v[:, :, keep], mask=np.ascontiguousarray(mask[:, :, keep]))
    assert np.allclose(a, b, rtol=0, atol=1e-12)


def pin_capacity_padding_is_invisible(orc):
    """Cache rows past sk (or past total_lengths) are never read: filling them with NaN, or
    dropping them from the allocation, changes nothing."""
    rng = _rng(507)
    B, Hkv, C, sk = 2, 2, 10, 7
    q = _randn(rng, B, 4, 5, 3)
    k, v = _randn(rng, B, Hkv, C, 3), _randn(rng, B, Hkv, C, 3)
    total = np.array([7, 4], np.int32)
    a = orc.forward(q, k[:, :, :sk].copy(), v[:, :, :sk].copy(), total_lengths=total)
    k2, v2 = k.copy(), v.copy()
    k2[:, :, sk:] = np.nan
    v2[:, :, sk:] = np.nan
    k2[1, :, 4:] = np.nan
    v2[1, :, 4:] = np.nan
    b = orc.forward(q, k2, v2, sk=sk, total_lengths=total)
    assert np.array_equal(a, b)


def pin_mask_plane_selection(orc):
    """Plane 0 for a single plane, plane b for B planes, plane b*H+h for B*H planes; each
    plane row i kills one key, seen as a zero in the probability row (V = identity)."""
    B, H, Hkv, Sq, C = 2, 4, 2, 3, 8
    rng = _rng(508)
    q, k = _randn(rng, B, H, Sq, C), _randn(rng, B, Hkv, C, C)
    v = np.broadcast_to(np.eye(C, dtype=np.float32), (B, Hkv, C, C)).copy()
    for planes in (1, B, B * H):
        mask = np.zeros((planes, Sq, C), np.float32)
        for p in range(planes):
            for i in range(Sq):
                mask[p, i, (p + 2 * i) % C] = -np.inf
        out = orc.forward(q, k, v, mask=mask)
        for b in range(B):
            for h in range(H):
                p = 0 if planes == 1 else (b if planes == B else b * H + h)
                for i in range(Sq):
                    row = out[b, h, i]
                    dead = (p + 2 * i) % C
                    assert row[dead] == 0.0, (planes, b, h, i)
                    assert np.all(np.delete(row, dead) > 0), (planes, b, h, i)


def pin_fully_masked_rows_are_zero(orc):
    rng = _rng(509)
    q, k, v = _randn(rng, 1, 2, 5, 4), _randn(rng, 1, 2, 6, 4), _randn(rng, 1, 2, 6, 4)
    mask = np.zeros((1, 5, 6), np.float32)
    mask[0, 1, :] = -np.inf
    mask[0, 3, :4] = -np.inf
    out = orc.forward(q, k, v, mask=mask, causal=True)
    # row 1 is killed by the mask; with causal (cmax = 1 + i), row 3 still sees key 4
    assert np.array_equal(out[0, :, 1], np.zeros((2, 4)))
    assert np.all(np.isfinite(out)) and np.any(out[0, :, 3] != 0)


def pin_rows_api_matches_forward(orc):
    rng = _rng(510)
    q, k, v = _randn(rng, 2, 4, 6, 5), _randn(rng, 2, 2, 9, 5), _randn(rng, 2, 2, 9, 5)
    kw = dict(causal=True, local_window=4, sk=8, total_lengths=np.array([8, 5], np.int32))
    full = orc.forward(q, k, v, **kw)
    picks = [(0, 0, 0), (1, 3, 5), (0, 2, 3), (1, 1, 0)]
    got = orc.rows(q, k, v, picks, **kw)
    for n, (b, h, i) in enumerate(picks):
        assert np.array_equal(got[n], full[b, h, i])


ALL_PINS = [obj for name, obj in sorted(globals().items()) if name.startswith("pin_")]
