"""GPU parity: the HIP kernels (through the C ABI) against the f64 oracle, element by element.

Tolerance: max-abs 1e-4 for fp32 inputs and 2e-2 for bf16/f16 inputs (fp32 accumulation);
rows with no attended finite key must be exactly 0.
"""

import math

import numpy as np
import pytest
import torch

import tiled_online_softmax_flash_amd as fa
import workloads
from gpu_util import TOL, check, oracle_full, run_gpu, say

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

NAMES = list(workloads.WORKLOADS)


@pytest.mark.parametrize("name", NAMES)
def test_small_workload_full_output(name):
    prob = workloads.workload(name, small=True)
    say(f"[gpu] small workload {name}: q{tuple(prob.q.shape)} k{tuple(prob.k.shape)} {prob.dtype}")
    got = run_gpu(prob, out_fill=float("nan")).double().cpu().numpy()
    want = oracle_full(prob)
    check(got, want, prob.dtype, name)
    if name in workloads.SPLITKV_WORKLOADS:   # also through the entry point bench.py times
        got = run_gpu(prob, out_fill=float("nan"), splitkv=True).double().cpu().numpy()
        check(got, want, prob.dtype, name + "/splitkv")


@pytest.mark.parametrize("name", NAMES)
def test_full_workload_full_output(name):
    """The whole output at full size, in the launch configuration bench.py times (the split-key
    entry point for the decode workload), element by element against the whole oracle output."""
    prob = workloads.workload(name)
    say(f"[gpu] full workload {name}: q{tuple(prob.q.shape)} k{tuple(prob.k.shape)} {prob.dtype}")
    out = run_gpu(prob, out_fill=float("nan"), splitkv=name in workloads.SPLITKV_WORKLOADS)
    assert bool(torch.isfinite(out).all()), "non-finite values in the output"
    if prob.mask is not None:
        # every (b, h) of a fully masked mask row is exactly zero
        dead = torch.nonzero(torch.isinf(prob.mask).all(dim=-1))  # (plane, i)
        assert len(dead) > 0
        for plane, i in dead.tolist():
            if prob.out_layout == "head":
                assert bool((out[plane, :, i] == 0).all())
    got = out.double().cpu().numpy()
    del out
    check(got, oracle_full(prob), prob.dtype, name)


# ------------------------------------------------------------------------------------------
# edge cases of the key rule and the epilogue

EDGE = {
    "window_one_past": dict(seed=21, batch=3, heads=4, kv_heads=2, sq=70, sk=300, dim=64,
                            dtype="bf16", causal=True, local_window=1, lengths="past",
                            max_past=200),
    "window_wider_than_keys": dict(seed=22, batch=2, heads=4, kv_heads=4, sq=130, sk=130, dim=64,
                                   dtype="f16", causal=True, local_window=5000),
    "past_zero_total_short": dict(seed=23, batch=2, heads=2, kv_heads=1, sq=200, sk=256,
                                  dim=128, dtype="bf16", causal=True, lengths="past", max_past=0),
    "queries_exceed_keys": dict(seed=24, batch=2, heads=2, kv_heads=2, sq=300, sk=70, dim=64,
                                dtype="bf16", causal=True),
    "total_only_random": dict(seed=25, batch=4, heads=2, kv_heads=1, sq=90, sk=333, dim=64,
                              dtype="f16", lengths="total"),
    "past_only": dict(seed=26, batch=3, heads=2, kv_heads=2, sq=65, sk=400, dim=64, dtype="bf16",
                      causal=True, lengths="past_only", max_past=300),
    "window_non_causal": dict(seed=27, batch=2, heads=2, kv_heads=1, sq=129, sk=260, dim=32,
                              dtype="bf16", local_window=70),
    "single_query_row": dict(seed=28, batch=2, heads=8, kv_heads=2, sq=1, sk=777, dim=128,
                             dtype="bf16", causal=True),
    "single_key": dict(seed=29, batch=1, heads=3, kv_heads=1, sq=40, sk=1, dim=64, dtype="f16"),
    "softcap_saturating": dict(seed=30, batch=2, heads=4, kv_heads=2, sq=150, sk=200, dim=64,
                               dtype="f16", softcap=2.0, amp=3.0, causal=True),
    # the largest softcap that takes the identity tanh, with small scores (where it has no
    # relative accuracy), and the next one up (the series near 0)
    "softcap_identity_limit": dict(seed=33, batch=1, heads=4, kv_heads=1, sq=130, sk=260, dim=128,
                                   dtype="bf16", softcap=1024.0, amp=0.3, causal=True),
    "softcap_above_identity_limit": dict(seed=34, batch=1, heads=4, kv_heads=1, sq=130, sk=260,
                                         dim=128, dtype="f16", softcap=1025.0, amp=0.3,
                                         causal=True),
    # a large cap with an additive mask (identity tanh, masked kernel) and one above the limit
    "softcap_1000_with_mask": dict(seed=35, batch=2, heads=2, kv_heads=2, sq=100, sk=96, dim=64,
                                   dtype="bf16", softcap=1000.0, amp=0.3, mask="normal",
                                   mask_p=0.2),
    "softcap_2000_with_mask": dict(seed=36, batch=2, heads=2, kv_heads=2, sq=100, sk=96, dim=128,
                                   dtype="f16", softcap=2000.0, amp=0.3, mask="bernoulli",
                                   mask_p=0.2),
    "softcap_huge_is_plain": dict(seed=31, batch=1, heads=2, kv_heads=1, sq=100, sk=100, dim=64,
                                  dtype="bf16", softcap=1e30),
    "softcap_with_mask": dict(seed=32, batch=2, heads=2, kv_heads=2, sq=100, sk=96, dim=64,
                              dtype="bf16", softcap=5.0, mask="normal", mask_p=0.2),
    "mask_single_plane": dict(seed=33, batch=2, heads=4, kv_heads=2, sq=77, sk=140, dim=64,
                              dtype="bf16", mask="bernoulli", mask_planes=1, mask_p=0.3,
                              dead_rows=2),
    "mask_per_head": dict(seed=34, batch=2, heads=3, kv_heads=3, sq=70, sk=130, dim=64,
                          dtype="f16", mask="normal", mask_planes=6, mask_p=0.1, dead_rows=1),
    "mask_bf16_values": dict(seed=35, batch=2, heads=2, kv_heads=1, sq=66, sk=192, dim=128,
                             dtype="bf16", mask="normal", mask_dtype="bf16", mask_p=0.1),
    "mask_ragged_sk": dict(seed=36, batch=1, heads=2, kv_heads=2, sq=50, sk=131, dim=64,
                           dtype="bf16", mask="normal", mask_p=0.1, causal=True),
    "mask_with_lengths": dict(seed=37, batch=3, heads=2, kv_heads=1, sq=40, sk=300, dim=64,
                              dtype="bf16", mask="bernoulli", mask_p=0.1, causal=True,
                              local_window=100, lengths="past", max_past=200,
                              nan_beyond_total=True),
    "capacity_beyond_sk": dict(seed=38, batch=2, heads=4, kv_heads=2, sq=100, sk=150,
                               kv_capacity=512, dim=128, dtype="bf16", causal=True),
    "scale_negative": dict(seed=39, batch=1, heads=2, kv_heads=1, sq=80, sk=120, dim=64,
                           dtype="bf16", scale=-0.2),
    "scale_zero": dict(seed=40, batch=1, heads=2, kv_heads=1, sq=80, sk=120, dim=64,
                       dtype="bf16", scale=0.0, causal=True),
    "token_major_batched": dict(seed=41, batch=3, heads=5, kv_heads=5, sq=70, sk=90, dim=64,
                                dtype="bf16", out_layout="token", causal=True),
    "token_major_fp32": dict(seed=42, batch=2, heads=3, kv_heads=1, sq=100, sk=100, dim=128,
                             dtype="f32", out_layout="token"),
    "fp32_gqa_causal_window": dict(seed=43, batch=2, heads=4, kv_heads=2, sq=150, sk=180,
                                   dim=64, dtype="f32", causal=True, local_window=50,
                                   lengths="past", max_past=30),
    "fp32_mask_softcap": dict(seed=44, batch=2, heads=2, kv_heads=2, sq=70, sk=100, dim=64,
                              dtype="f32", mask="bernoulli", mask_p=0.2, dead_rows=3,
                              softcap=3.0),
    "amp3_bf16_causal": dict(seed=45, batch=1, heads=4, kv_heads=1, sq=300, sk=300, dim=128,
                             dtype="bf16", causal=True, amp=3.0),
    # 256-row kernel, head dim 128, token-major rows written through the output staging, last
    # query tile ragged
    "token_major_d128_ragged": dict(seed=46, batch=2, heads=8, kv_heads=2, sq=600, sk=600,
                                    dim=128, dtype="bf16", out_layout="token", causal=True),
    # 768 work items: every persistent workgroup runs several, with the next item's tiles and Q
    # loaded during the current one's last steps; ragged last query tile
    "many_items_per_workgroup": dict(seed=47, batch=8, heads=32, kv_heads=8, sq=520, sk=520,
                                     dim=128, dtype="bf16", causal=True),
    # fp32 head dims 129..384 (four 96-dim groups; dims past D in the last groups unused)
    "fp32_d384_gqa_causal_lengths": dict(seed=50, batch=2, heads=4, kv_heads=2, sq=150, sk=170,
                                         dim=384, dtype="f32", causal=True, lengths="past",
                                         max_past=20),
    "fp32_d200_window": dict(seed=51, batch=1, heads=3, kv_heads=1, sq=100, sk=260, dim=200,
                             dtype="f32", causal=True, local_window=70),
    "fp32_d300_mask_softcap": dict(seed=52, batch=2, heads=2, kv_heads=2, sq=70, sk=100, dim=300,
                                   dtype="f32", mask="bernoulli", mask_p=0.2, dead_rows=3,
                                   softcap=3.0),
    "fp32_d129_token_major": dict(seed=53, batch=2, heads=3, kv_heads=3, sq=65, sk=65, dim=129,
                                  dtype="f32", out_layout="token"),
    # the fp32 key-split form (small problems take it): one key tile, so the second key half
    # has nothing to do; causal rows whose keys all fall in the first half; a window narrower
    # than a tile, where each half holds keys for some row groups only; a ragged 32-row tile
    "fp32_split_one_key_tile": dict(seed=95, batch=1, heads=2, kv_heads=1, sq=45, sk=10, dim=64,
                                    dtype="f32"),
    "fp32_split_causal_odd_tiles": dict(seed=96, batch=2, heads=2, kv_heads=2, sq=83, sk=83,
                                        dim=128, dtype="f32", causal=True),
    "fp32_split_narrow_window": dict(seed=97, batch=1, heads=3, kv_heads=1, sq=100, sk=140,
                                     dim=32, dtype="f32", causal=True, local_window=9),
    # 256 tiles of 64 rows: on 256 CUs the fp32 kernel keeps whole 64-row workgroups here (the
    # key-split form takes the other fp32 cases: too few tiles, or a fractional number per CU)
    "fp32_d128_whole_tiles": dict(seed=94, batch=1, heads=8, kv_heads=8, sq=2048, sk=150, dim=128,
                                  dtype="f32", causal=True),
    # wide fp32 head dims on whole 64-dim runs below 384 (the K dims past them are never loaded)
    # and a 16-dim-aligned one, with an additive mask and no softcap
    "fp32_d256_mask": dict(seed=91, batch=1, heads=3, kv_heads=1, sq=90, sk=150, dim=256,
                           dtype="f32", mask="bernoulli", mask_p=0.3, dead_rows=2),
    "fp32_d192_causal_ragged": dict(seed=92, batch=2, heads=2, kv_heads=1, sq=97, sk=131, dim=192,
                                    dtype="f32", causal=True),
    "fp32_d336_long": dict(seed=93, batch=1, heads=1, kv_heads=1, sq=64, sk=700, dim=336,
                           dtype="f32"),
    # scores that drift by hundreds along the keys (rising for some rows, falling for others):
    # later half-tiles exceed the running maximum far beyond the lazy-rescale bound, and their
    # weights against the old maximum overflow fp32 (head dims 128 and 64, with and without a
    # causal rule, a softcap that keeps them bounded, and an additive mask that ramps up)
    "key_ramp_bf16_d128": dict(seed=54, batch=2, heads=4, kv_heads=2, sq=300, sk=520, dim=128,
                               dtype="bf16", key_ramp=0.5),
    "key_ramp_f16_d64_causal": dict(seed=55, batch=2, heads=4, kv_heads=1, sq=520, sk=520, dim=64,
                                    dtype="f16", key_ramp=0.25, causal=True),
    "key_ramp_bf16_d128_softcap": dict(seed=56, batch=1, heads=4, kv_heads=2, sq=260, sk=400,
                                       dim=128, dtype="bf16", key_ramp=0.5, softcap=30.0),
    "mask_ramp_bf16_d64": dict(seed=57, batch=2, heads=2, kv_heads=2, sq=300, sk=512, dim=64,
                               dtype="bf16", mask="ramp", mask_ramp=0.75, mask_p=0.1),
    # masks at the end of the float32 range: rows whose attended keys all hold the most
    # negative finite value get a uniform softmax (not zeros), and that value loses to 0 or to
    # half of it; the running maximum sits near -3.4e38, where its exponent offset overflows
    "mask_extreme_bf16_d64": dict(seed=59, batch=2, heads=2, kv_heads=1, sq=90, sk=300, dim=64,
                                  dtype="bf16", mask="extreme", mask_p=0.05, causal=True),
    "mask_extreme_f16_d128": dict(seed=60, batch=1, heads=3, kv_heads=3, sq=70, sk=200, dim=128,
                                  dtype="f16", mask="extreme", mask_p=0.05),
    "mask_extreme_bf16_d96_bf16mask": dict(seed=61, batch=2, heads=2, kv_heads=2, sq=60, sk=160,
                                           dim=96, dtype="bf16", mask="extreme", mask_p=0.05,
                                           mask_dtype="bf16"),
    "mask_extreme_fp32": dict(seed=62, batch=1, heads=2, kv_heads=1, sq=50, sk=130, dim=64,
                              dtype="f32", mask="extreme", mask_p=0.05),
    # masked bf16 head dim 64 with a power-of-two scale and an fp32 mask: Q takes the scale and
    # the Q.K products start from the mask values; a 16-bit mask, or a scale that is not a power
    # of two, keeps the per-score multiply-add
    "mask_acc_scale_one_bf16_d64": dict(seed=64, batch=2, heads=3, kv_heads=3, sq=200, sk=330,
                                        dim=64, dtype="bf16", scale=1.0, amp=0.3, mask="normal",
                                        mask_p=0.1, dead_rows=2),
    "mask_acc_per_head_planes_bf16_d64": dict(seed=71, batch=2, heads=3, kv_heads=3, sq=100,
                                              sk=200, dim=64, dtype="bf16", mask="normal",
                                              mask_planes=6, mask_p=0.1, dead_rows=1),
    "mask_pow2_scale_bf16mask": dict(seed=65, batch=2, heads=2, kv_heads=1, sq=150, sk=260,
                                        dim=64, dtype="bf16", scale=2.0 ** -5, mask="ramp",
                                        mask_ramp=0.25, mask_p=0.1, mask_dtype="bf16", causal=True),
    # softcaps at which many scores straddle |s / c| = 1/8, where the speculative softmax's
    # polynomial form of c tanh(s / c) ends and rows are redone with the exact form
    "softcap_series_edge_f16_d128": dict(seed=67, batch=2, heads=4, kv_heads=2, sq=300, sk=400,
                                         dim=128, dtype="f16", softcap=8.0, causal=True),
    "softcap_series_edge_bf16_d64": dict(seed=68, batch=2, heads=4, kv_heads=1, sq=280, sk=520,
                                         dim=64, dtype="bf16", softcap=4.0, causal=True,
                                         local_window=200),
    # the softcap's polynomial exponent with a negative scale (odd coefficients change sign) and
    # with a zero scale (every score 0: uniform weights)
    "softcap_negative_scale_f16_d128": dict(seed=69, batch=2, heads=2, kv_heads=1, sq=150, sk=260,
                                            dim=128, dtype="f16", softcap=6.0, scale=-0.3,
                                            causal=True),
    "softcap_zero_scale_bf16_d64": dict(seed=70, batch=1, heads=3, kv_heads=3, sq=90, sk=200,
                                        dim=64, dtype="bf16", softcap=20.0, scale=0.0),
    "mask_fma_scale_0p1_bf16_d64": dict(seed=66, batch=2, heads=2, kv_heads=2, sq=140, sk=300,
                                        dim=64, dtype="bf16", scale=0.1, mask="normal", mask_p=0.1,
                                        dead_rows=1),
    # fp32: scores that keep rising along the keys make the running maximum stale tile after
    # tile (the kernel's exact redo; the ramp keeps the scores' own fp32 rounding, about 2e-5 in
    # the output, inside the gate).  Zero queries with masks offset by thousands make the scores
    # the exact mask values at |m log2 e| above 4096, where the weights are formed by
    # subtracting before scaling.
    "key_ramp_fp32_d128": dict(seed=63, batch=2, heads=4, kv_heads=2, sq=300, sk=520, dim=128,
                               dtype="f32", key_ramp=0.05),
    "key_ramp_fp32_d64_causal_softcap": dict(seed=64, batch=1, heads=4, kv_heads=2, sq=330,
                                             sk=330, dim=64, dtype="f32", key_ramp=0.25,
                                             causal=True, softcap=30.0),
    "mask_offset_fp32_d128_ramp": dict(seed=65, batch=1, heads=3, kv_heads=3, sq=130, sk=512,
                                       dim=128, dtype="f32", mask="ramp", mask_ramp=0.002,
                                       mask_offset=3000.0, mask_p=0.1, q_scale=0.0),
    "mask_offset_fp32_d72_causal": dict(seed=66, batch=2, heads=2, kv_heads=1, sq=200, sk=300,
                                        dim=72, dtype="f32", mask="normal", mask_offset=-6000.0,
                                        mask_p=0.05, causal=True, q_scale=0.0),
    "mask_ramp_fp32_d72": dict(seed=67, batch=2, heads=2, kv_heads=1, sq=200, sk=300, dim=72,
                               dtype="f32", mask="ramp", mask_ramp=0.75, mask_p=0.05,
                               causal=True),
    "mask_ramp_f16_d128_f16mask": dict(seed=58, batch=2, heads=2, kv_heads=1, sq=200, sk=448,
                                        dim=128, dtype="f16", mask="ramp", mask_ramp=0.5,
                                        mask_p=0.05, mask_planes=1, mask_dtype="f16"),
}


@pytest.mark.parametrize("name", list(EDGE))
def test_edge_case(name):
    prob = workloads.make_problem(name=name, **EDGE[name])
    say(f"[gpu] edge {name}: q{tuple(prob.q.shape)} k{tuple(prob.k.shape)} sk={prob.sk} {prob.dtype}")
    got = run_gpu(prob, out_fill=float("nan")).double().cpu().numpy()
    check(got, oracle_full(prob), prob.dtype, name, amp=EDGE[name].get("amp", 1.0))


# ------------------------------------------------------------------------------------------
# key-rule edges that the workloads never reach (their lengths keep total = past + Sq <= Sk),
# for every kernel family.  The rule is that of flash_attention_body on the flash_attention.rs
# page: logical length capped at sk, causal limit past + i (else L - Sq + i), window start
# causal limit + 1 - W.

KEY_RULE = {
    # past and total drawn independently, total up to the capacity: rows whose causal limit
    # passes L - 1, batches whose total is below their past, totals past sk (rows >= sk NaN)
    "indep_causal": dict(causal=True, lengths="indep", max_past=500, nan_beyond_total=True),
    # the same with a window: rows whose window starts past L - 1 attend nothing
    "indep_causal_window": dict(causal=True, local_window=48, lengths="indep", max_past=500,
                                nan_beyond_total=True),
    # total above sk (below the capacity) without past lengths: L capped at sk and the causal
    # base L - Sq; cache rows at and past sk are NaN
    "total_beyond_sk": dict(causal=True, lengths="explicit", total_values=[640, 512, 301, 0],
                            nan_beyond_total=True, sk=300),
    # zero and negative lengths, with a window
    "zero_and_negative_lengths": dict(causal=True, local_window=100, lengths="explicit",
                                      total_values=[0, -7, 250, 400],
                                      past_values=[-5, 3, -300, 390], nan_beyond_total=True),
}

FAMILIES = {
    "ring_bf16_d128": dict(dtype="bf16", dim=128),
    "ring_f16_d64": dict(dtype="f16", dim=64),
    "fwd16_bf16_d96": dict(dtype="bf16", dim=96),
    # contiguous but not 16-byte aligned: the ring kernel's alignment gate sends these to fwd16
    "fwd16_misaligned_f16_d128": dict(dtype="f16", dim=128, misalign=True),
    "fwd16_misaligned_bf16_d64": dict(dtype="bf16", dim=64, misalign=True),
    "fp32_d64": dict(dtype="f32", dim=64),
    "fp32_misaligned_d128": dict(dtype="f32", dim=128, misalign=True),
    "fp32_wide_d200": dict(dtype="f32", dim=200),
    # the wide kernel's straight-line tile loads (head dim 384), and its looped ones from
    # pointers that are 4- but not 16-byte aligned
    "fp32_wide_d384": dict(dtype="f32", dim=384),
    "fp32_wide_misaligned_d256": dict(dtype="f32", dim=256, misalign=True),
}


@pytest.mark.parametrize("family", list(FAMILIES))
@pytest.mark.parametrize("rule", list(KEY_RULE))
def test_key_rule_edges(rule, family):
    fam = dict(FAMILIES[family])
    misalign = fam.pop("misalign", False)
    params = dict(seed=100 + list(KEY_RULE).index(rule), batch=4, heads=8, kv_heads=2, sq=300,
                  sk=400, kv_capacity=640, **fam)
    params.update(KEY_RULE[rule])
    prob = workloads.make_problem(name=f"{rule}-{family}", **params)
    say(f"[gpu] key rule {rule} / {family}: q{tuple(prob.q.shape)} sk={prob.sk} "
        f"total={None if prob.total_lengths is None else prob.total_lengths.tolist()} "
        f"past={None if prob.past_lengths is None else prob.past_lengths.tolist()} misalign={misalign}")
    want = oracle_full(prob)
    got = run_gpu(prob, out_fill=float("nan"), misalign=misalign).double().cpu().numpy()
    check(got, want, prob.dtype, f"{rule}-{family}")
    assert _edge_reached(prob, rule), f"{rule}: the inputs do not reach the edge"


def _edge_reached(prob, rule) -> bool:
    """Whether the drawn lengths reach the edge the case is named for (a property of the
    inputs, counted from the stated rule)."""
    total = prob.total_lengths.tolist()
    past = None if prob.past_lengths is None else prob.past_lengths.tolist()
    if rule == "total_beyond_sk":
        return any(t > prob.sk for t in total)
    if rule == "zero_and_negative_lengths":
        return min(total) <= 0 and min(past) < 0
    over = window_past_end = 0
    for b in range(prob.batch):
        L = max(min(total[b], prob.sk), 0)
        cmax_last = past[b] + prob.sq - 1
        over += cmax_last > L - 1
        window_past_end += prob.local_window > 0 and cmax_last + 1 - prob.local_window > L - 1
    return over > 0 and (prob.local_window == 0 or window_past_end > 0)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("dim", [1, 8, 40, 64, 72, 100, 128])
def test_head_dims(dtype, dim):
    prob = workloads.make_problem(name=f"dim{dim}", seed=50 + dim, batch=2, heads=4, kv_heads=2,
                                  sq=133, sk=161, dim=dim, dtype=dtype, causal=True)
    say(f"[gpu] head dim {dim} {dtype}")
    got = run_gpu(prob, out_fill=float("nan")).double().cpu().numpy()
    check(got, oracle_full(prob), dtype, f"dim{dim}-{dtype}")


def test_f16_relative_error_across_amplitudes():
    """Relative error with a floored denominator stays at the fp16 rounding floor at unit and
    larger input magnitudes: the accumulators must be fp32.  This is the amplitude sweep of the
    parity test on the onnx-runtime-ep-cuda page src/kernels/flash_attention.rs, with its
    one-signed input range ([-1, 0) times the amplitude) and its gates (2e-3 absolute at unit
    amplitude, 6e-3 relative with the denominator floored at 1e-2)."""
    worst_rel = 0.0
    for amp in (1.0, 3.0):
        for seq in (2, 30, 64, 96, 192, 300):
            prob = workloads.make_problem(name="amp", seed=60 + seq, batch=1, heads=14,
                                          kv_heads=2, sq=seq, sk=seq, dim=64, dtype="f16",
                                          causal=True, amp=amp, dist="neg_uniform")
            say(f"[gpu] f16 amplitude {amp} seq {seq}")
            got = run_gpu(prob).double().cpu().numpy()
            want = oracle_full(prob)
            err = np.abs(got - want)
            worst_rel = max(worst_rel, float((err / np.maximum(np.abs(want), 1e-2)).max()))
            if amp == 1.0:
                assert err.max() < 2e-3
    say(f"  worst relative error {worst_rel:.3e}")
    assert worst_rel < 6e-3


def test_no_keys_writes_zeros():
    prob = workloads.make_problem(name="nokeys", seed=70, batch=2, heads=4, kv_heads=2, sq=50,
                                  sk=0, kv_capacity=0, dim=64, dtype="bf16")
    say("[gpu] sk = 0")
    out = run_gpu(prob, out_fill=float("nan"))
    assert bool((out == 0).all())


def test_lengths_all_zero_writes_zeros():
    prob = workloads.make_problem(name="zerolen", seed=71, batch=2, heads=2, kv_heads=2, sq=64,
                                  sk=64, dim=64, dtype="f16")
    prob.total_lengths = torch.zeros(2, dtype=torch.int32)
    say("[gpu] total_lengths = 0")
    out = run_gpu(prob, out_fill=float("nan"))
    assert bool((out == 0).all())


def test_empty_problem_is_a_no_op():
    q = torch.empty(0, 4, 16, 64, dtype=torch.bfloat16, device="cuda")
    kv = torch.empty(0, 2, 16, 64, dtype=torch.bfloat16, device="cuda")
    say("[gpu] empty batch")
    out = fa.flash_attn_fwd(q, kv, kv)
    assert out.shape == (0, 4, 16, 64)


def test_side_stream_and_out_argument():
    prob = workloads.workload("gqa_causal", small=True)
    d = prob.to("cuda")
    out = torch.full_like(d.q, float("nan"))
    s = torch.cuda.Stream()
    say("[gpu] side stream")
    with torch.cuda.stream(s):
        res = fa.flash_attn_fwd(d.q, d.k, d.v, out=out, **d.kwargs())
    s.synchronize()
    assert res.data_ptr() == out.data_ptr()
    check(out.double().cpu().numpy(), oracle_full(prob), prob.dtype, "side-stream")


def test_concurrent_streams_do_not_interfere():
    # the kernels keep no state between calls: four problems (the 256-row ring kernel with and
    # without a mask, the fp32 kernel in its key-split form, the wide fp32 kernel) run on four
    # streams at once, three times each, and every result equals a lone call's bit for bit
    names = ["gqa_causal", "masked_long", "dit_joint", "vae_decoder"]
    devs = [workloads.workload(n, small=True).to("cuda") for n in names]
    say("[gpu] concurrent streams: " + ", ".join(names))
    refs = [fa.flash_attn_fwd(d.q, d.k, d.v, **d.kwargs()) for d in devs]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in devs]
    outs = [[] for _ in devs]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        for i, (d, s) in enumerate(zip(devs, streams)):
            with torch.cuda.stream(s):
                outs[i].append(fa.flash_attn_fwd(d.q, d.k, d.v, **d.kwargs()))
    torch.cuda.synchronize()
    for name, ref, got in zip(names, refs, outs):
        for o in got:
            assert torch.equal(o, ref), name


def test_repeated_calls_are_deterministic():
    prob = workloads.workload("masked_long", small=True)
    say("[gpu] determinism")
    a = run_gpu(prob)
    b = run_gpu(prob)
    assert torch.equal(a, b)


def test_gpu_rejects_noncontiguous_input():
    q = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16, device="cuda").transpose(1, 2)
    with pytest.raises(ValueError):
        fa.flash_attn_fwd(q, q, q)
