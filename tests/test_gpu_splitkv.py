"""Split-key path (flash_attn_fwd_splitkv) against the oracle and against flash_attn_fwd.

Decode-shaped problems: one or a few query rows per sequence, every head of a GQA group in one
32-row block, long and ragged key ranges cut into spans whose partial softmax states a second
kernel merges, with and without additive masks.  Each case runs with the device's suggested number of spans and with a fixed
small and large one (spans past the key range hold no keys and must drop out of the merge).
"""

import pytest
import torch

import tiled_online_softmax_flash_amd as fa
import workloads
from gpu_util import check, oracle_full, say

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

CASES = {
    # one decode step per sequence, 4 query heads per KV head, ragged cache lengths
    "bf16_d128_decode_total": dict(seed=70, batch=3, heads=8, kv_heads=2, sq=1, sk=1000, dim=128,
                                   dtype="bf16", causal=True, lengths="total",
                                   nan_beyond_total=True),
    # cache of past rows plus this call's rows, 8 heads x 4 rows = one full 32-row block
    "bf16_d128_past_32rows": dict(seed=71, batch=2, heads=16, kv_heads=2, sq=4, sk=700,
                                  kv_capacity=704, dim=128, dtype="bf16", causal=True,
                                  lengths="past", max_past=690, nan_beyond_total=True),
    # f16, head dim 64, softcap and a local window
    "f16_d64_softcap_window": dict(seed=72, batch=2, heads=4, kv_heads=1, sq=2, sk=900, dim=64,
                                   dtype="f16", causal=True, local_window=300, softcap=30.0),
    # no causal rule, token-major output, GQA group of 1 (8 heads each with its own KV head)
    "bf16_d64_token_major": dict(seed=73, batch=1, heads=8, kv_heads=8, sq=3, sk=333, dim=64,
                                 dtype="bf16", out_layout="token"),
    # past lengths only (total = sk); a window shorter than a span
    "f16_d128_past_only_window": dict(seed=74, batch=2, heads=4, kv_heads=2, sq=1, sk=2048,
                                      dim=128, dtype="f16", causal=True, lengths="past_only",
                                      max_past=2047, local_window=40),
    # additive masks: one plane per batch (float32, -inf holes), per head (input dtype, with
    # softcap and fully masked rows), and a single plane with past lengths
    "bf16_d128_mask_batch_planes": dict(seed=76, batch=2, heads=8, kv_heads=2, sq=1, sk=700,
                                        dim=128, dtype="bf16", causal=True, mask="normal",
                                        mask_p=0.2),
    "f16_d64_mask_head_planes_softcap": dict(seed=77, batch=2, heads=4, kv_heads=2, sq=2, sk=500,
                                             dim=64, dtype="f16", mask="bernoulli", mask_p=0.3,
                                             mask_planes=8, mask_dtype="f16", softcap=20.0,
                                             dead_rows=1),
    "bf16_d128_mask_one_plane_past": dict(seed=78, batch=3, heads=16, kv_heads=2, sq=4, sk=600,
                                          dim=128, dtype="bf16", causal=True, lengths="past",
                                          max_past=590, mask="normal", mask_planes=1, dead_rows=1),
    # token-major output with a bf16 mask per head and a window
    "bf16_d64_token_major_head_mask": dict(seed=79, batch=2, heads=6, kv_heads=3, sq=3, sk=450,
                                           dim=64, dtype="bf16", out_layout="token", causal=True,
                                           local_window=200, mask="normal", mask_planes=12,
                                           mask_dtype="bf16", dead_rows=1),
    # keys fewer than one tile, and total lengths of 0 (fully masked rows)
    "bf16_d128_short": dict(seed=75, batch=4, heads=4, kv_heads=1, sq=1, sk=20, dim=128,
                            dtype="bf16", lengths="total"),
    # key-rule edges: past and total drawn independently (total up to the capacity, so causal
    # limits pass L - 1 and totals pass sk; cache rows at and past min(total, sk) are NaN)
    "bf16_d128_indep_lengths": dict(seed=150, batch=4, heads=8, kv_heads=2, sq=2, sk=700,
                                    kv_capacity=900, dim=128, dtype="bf16", causal=True,
                                    lengths="indep", max_past=800, nan_beyond_total=True),
    # totals above sk without past lengths (L capped at sk, causal base L - sq), with a window
    "f16_d64_total_beyond_sk_window": dict(seed=151, batch=4, heads=4, kv_heads=2, sq=3, sk=500,
                                           kv_capacity=768, dim=64, dtype="f16", causal=True,
                                           local_window=200, lengths="explicit",
                                           total_values=[768, 600, 501, 17],
                                           nan_beyond_total=True),
    # zero and negative lengths; windows that start past the length
    "bf16_d64_zero_negative_lengths": dict(seed=152, batch=4, heads=8, kv_heads=2, sq=2, sk=1000,
                                           dim=64, dtype="bf16", causal=True, local_window=64,
                                           lengths="explicit", total_values=[0, -4, 300, 1000],
                                           past_values=[-3, 5, 900, 995], nan_beyond_total=True),
}


def _kwargs(prob):
    return prob.to("cuda").kwargs()


@pytest.mark.parametrize("splits", [None, 4, 64])
@pytest.mark.parametrize("name", list(CASES))
def test_splitkv_parity(name, splits):
    prob = workloads.make_problem(name=name, **CASES[name])
    d = prob.to("cuda")
    kw = _kwargs(prob)
    say(f"[gpu] splitkv {name} splits={splits}: q{tuple(prob.q.shape)} k{tuple(prob.k.shape)} {prob.dtype}")
    got = fa.flash_attn_fwd_splitkv(d.q, d.k, d.v, num_splits=splits, **kw)
    torch.cuda.synchronize()
    check(got.double().cpu().numpy(), oracle_full(prob), prob.dtype, f"{name}/{splits}")
    # the single-pass kernel on the same inputs: both within tolerance of the oracle, and of
    # each other by at most twice that
    ref = fa.flash_attn_fwd(d.q, d.k, d.v, **kw)
    torch.cuda.synchronize()
    diff = (got.double() - ref.double()).abs().max().item()
    assert diff <= 2 * 2e-2, f"split-key vs single-pass: {diff:.3e}"


def test_splitkv_workspace_reuse_and_fill():
    """A caller workspace is overwritten, not accumulated into: garbage in it changes nothing,
    and a second call with fewer spans on the same workspace gives the same output."""
    prob = workloads.make_problem(name="reuse", **CASES["bf16_d128_decode_total"])
    d = prob.to("cuda")
    kw = _kwargs(prob)
    need = fa.splitkv_workspace_bytes(prob.batch, prob.kv_heads, prob.dim, 32)
    ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device="cuda")
    say("[gpu] splitkv workspace reuse")
    a = fa.flash_attn_fwd_splitkv(d.q, d.k, d.v, num_splits=32, workspace=ws, **kw).clone()
    b = fa.flash_attn_fwd_splitkv(d.q, d.k, d.v, num_splits=8, workspace=ws, **kw).clone()
    torch.cuda.synchronize()
    want = oracle_full(prob)
    check(a.double().cpu().numpy(), want, "bf16", "ws32")
    check(b.double().cpu().numpy(), want, "bf16", "ws8")


def test_splitkv_empty_cache_writes_zeros():
    prob = workloads.make_problem(name="empty", seed=76, batch=2, heads=4, kv_heads=2, sq=1, sk=0,
                                  kv_capacity=32, dim=64, dtype="bf16")
    d = prob.to("cuda")
    out = torch.full((2, 4, 1, 64), float("nan"), dtype=torch.bfloat16, device="cuda")
    say("[gpu] splitkv sk=0")
    fa.flash_attn_fwd_splitkv(d.q, d.k, d.v, out=out, num_splits=4, **_kwargs(prob))
    torch.cuda.synchronize()
    assert torch.all(out == 0).item()


def test_splitkv_graph_replay():
    """Both kernels of a call captured into a HIP graph; replays after eager work match."""
    prob = workloads.make_problem(name="graph", **CASES["bf16_d128_past_32rows"])
    d = prob.to("cuda")
    kw = _kwargs(prob)
    splits = fa.splitkv_suggested_splits(prob.batch, prob.kv_heads, prob.sk)
    ws = torch.empty(fa.splitkv_workspace_bytes(prob.batch, prob.kv_heads, prob.dim, splits),
                     dtype=torch.uint8, device="cuda")
    say(f"[gpu] splitkv graph replay, {splits} spans")
    out = fa.flash_attn_fwd_splitkv(d.q, d.k, d.v, num_splits=splits, workspace=ws, **kw)
    torch.cuda.synchronize()
    eager = out.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fa.flash_attn_fwd_splitkv(d.q, d.k, d.v, out=out, num_splits=splits, workspace=ws, **kw)
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(float("nan"))
        ws.fill_(255)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep} differs from the eager call"
    check(out.double().cpu().numpy(), oracle_full(prob), "bf16", "graph")


def test_splitkv_on_a_side_stream():
    prob = workloads.make_problem(name="side", **CASES["f16_d64_softcap_window"])
    d = prob.to("cuda")
    kw = _kwargs(prob)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())   # inputs were copied on the default stream
    say("[gpu] splitkv side stream")
    with torch.cuda.stream(side):
        out = fa.flash_attn_fwd_splitkv(d.q, d.k, d.v, num_splits=8, stream=side, **kw)
    side.synchronize()
    check(out.double().cpu().numpy(), oracle_full(prob), prob.dtype, "side-stream")


def test_splitkv_side_stream_not_current_keeps_workspace(monkeypatch):
    """stream= names a stream that is not the current one: the workspace the binding allocates
    must not be handed to work on the current stream before the side stream's kernels ran."""
    from gpu_util import AllocSpy, busy_stream, churn_hits

    prob = workloads.make_problem(name="side2", **CASES["bf16_d128_decode_total"])
    d = prob.to("cuda")
    kw = d.kwargs()
    splits = 8
    need = fa.splitkv_workspace_bytes(prob.batch, prob.kv_heads, prob.dim, splits)
    side = busy_stream()
    spy = AllocSpy()
    say("[gpu] splitkv on a side stream that is not current, allocations churned meanwhile")
    monkeypatch.setattr(torch, "empty", spy)
    out = fa.flash_attn_fwd_splitkv(d.q, d.k, d.v, num_splits=splits, stream=side, **kw)
    monkeypatch.undo()
    assert spy.ptrs, "the binding allocated nothing"
    hits = churn_hits(spy.ptrs - {out.data_ptr()}, need)
    side.synchronize()
    assert hits == 0, "the workspace was reused while the side stream still needed it"
    check(out.double().cpu().numpy(), oracle_full(prob), prob.dtype, "side-stream-not-current")
