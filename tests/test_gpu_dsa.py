"""Sparse index selection (dsa_index_select) on the GPU against the oracle: the selected positions
must be identical, and so must every cell's score (read back from the workspace, which holds one
total-order key per cell, 0 for a removed position)."""

import numpy as np
import pytest
import torch

import tiled_online_softmax_flash_amd as fa
import workloads
from gpu_util import say
from oracle import dsa as dsa_oracle

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

CASES = {
    # decode rows: one query row per sequence, every position allowed
    "bf16_decode_d128": dict(seed=80, batch=2, q_seq=1, heads=8, head_dim=128, key_seq=3000,
                             top_k=512, dtype="bf16"),
    # a prefill chunk whose early rows allow fewer positions than top_k (-1 padding)
    "f16_chunk_padding": dict(seed=81, batch=1, q_seq=20, heads=4, head_dim=64, key_seq=100,
                              top_k=90, dtype="f16"),
    # fp32, odd head dim, random finite bias with -inf holes, ragged last tile
    "f32_d33_random_bias": dict(seed=82, batch=2, q_seq=3, heads=3, head_dim=33, key_seq=517,
                                top_k=40, dtype="f32", bias="random", hole_p=0.2,
                                weights_scale=0.5, scale=0.3),
    # small integers: many exactly tied scores, ties must go to the lower position
    "bf16_ties": dict(seed=83, batch=2, q_seq=2, heads=2, head_dim=8, key_seq=700, top_k=100,
                      dtype="bf16", bias="zero", int_values=True, scale=1.0),
    # overflowing products: +-inf and NaN scores (NaN canonical, the largest)
    "bf16_overflow": dict(seed=84, batch=1, q_seq=2, heads=8, head_dim=16, key_seq=300, top_k=20,
                          dtype="bf16", bias="random", overflow_keys=25),
    "f16_overflow_inf_keys": dict(seed=85, batch=1, q_seq=1, heads=4, head_dim=32, key_seq=200,
                                  top_k=30, dtype="f16", overflow_keys=10),
    # top_k wider than the key range; one head of one dim
    "f32_topk_wider_than_keys": dict(seed=86, batch=3, q_seq=1, heads=1, head_dim=1, key_seq=50,
                                     top_k=64, dtype="f32"),
    # no heads: every score is the bias
    "f32_no_heads": dict(seed=87, batch=1, q_seq=2, heads=0, head_dim=16, key_seq=300, top_k=10,
                         dtype="f32", bias="random"),
    # a long row: 20 chunks of 2048 positions
    "bf16_uncached_long": dict(seed=90, batch=1, q_seq=2, heads=2, head_dim=32, key_seq=40000,
                               top_k=1000, dtype="bf16", bias="random", hole_p=0.1),
    # every score equal (no heads, zero bias): every radix digit of every position matches the
    # threshold's, and the winners are the lowest positions, all ties, over 5 and 2 chunks
    "f32_all_equal_9000": dict(seed=94, batch=1, q_seq=2, heads=0, head_dim=16, key_seq=9000,
                               top_k=3000, dtype="f32", bias="zero"),
    "f32_all_equal_4000": dict(seed=95, batch=1, q_seq=2, heads=0, head_dim=16, key_seq=4000,
                               top_k=1500, dtype="f32", bias="zero"),
    # ties at the threshold spread over several 2048-position chunks of a row (integer inputs:
    # a handful of distinct scores), and a multi-chunk row with fewer allowed positions than
    # top_k (-1 padding after winners from every chunk)
    "bf16_ties_many_chunks": dict(seed=92, batch=2, q_seq=2, heads=2, head_dim=8, key_seq=9000,
                                  top_k=3000, dtype="bf16", bias="zero", int_values=True,
                                  scale=1.0),
    "f16_multichunk_padding": dict(seed=93, batch=1, q_seq=3, heads=4, head_dim=16, key_seq=5000,
                                   top_k=4500, dtype="f16", bias="random", hole_p=0.2),
    # many rows and a long key range
    "bf16_rows_long": dict(seed=88, batch=2, q_seq=5, heads=16, head_dim=128, key_seq=8192,
                           top_k=2048, dtype="bf16"),
}


def _order_keys(scores: np.ndarray, allowed: np.ndarray) -> np.ndarray:
    u = scores.astype(np.float32).view(np.uint32)
    k = np.where(u & 0x80000000, ~u, u | 0x80000000).astype(np.uint32)
    return np.where(allowed.astype(bool), k, 0).astype(np.uint32)


def _run(prob, workspace=None):
    d = prob.to("cuda")
    B, S, H, D = prob.query.shape
    T = prob.key.shape[1]
    if workspace is None:
        workspace = torch.full((max(fa.dsa_workspace_bytes(B, S, T), 4) // 4,), 0x5A5A5A5A,
                               dtype=torch.int32, device="cuda")
    out = torch.full((B, 1, S, prob.top_k), -7, dtype=torch.int64, device="cuda")
    fa.dsa_index_select(d.query, d.key, d.weights, d.bias, out=out, workspace=workspace,
                        **prob.kwargs())
    torch.cuda.synchronize()
    return out.cpu().numpy(), workspace


@pytest.mark.parametrize("name", list(CASES))
def test_dsa_matches_oracle_exactly(name):
    prob = workloads.make_dsa_problem(name=name, **CASES[name])
    B, S, H, D = prob.query.shape
    T = prob.key.shape[1]
    say(f"[gpu] dsa {name}: q{tuple(prob.query.shape)} k{tuple(prob.key.shape)} top_k {prob.top_k} {prob.dtype}")
    got, ws = _run(prob)
    sc, al = dsa_oracle.scores(prob.query, prob.key, prob.weights, prob.bias, scale=prob.scale,
                               weights_scale=prob.weights_scale)
    want = dsa_oracle.select(sc, al, prob.top_k)
    if T:
        keys = ws[: B * S * T].cpu().numpy().view(np.uint32).reshape(B, S, T)
        ref = _order_keys(sc, al)
        bad = np.nonzero(keys != ref)
        assert bad[0].size == 0, f"{bad[0].size} cells differ, first at {tuple(int(x[0]) for x in bad)}"
    assert np.array_equal(got, want), f"{int((got != want).sum())} selected positions differ"
    say(f"  {name}: {int((got >= 0).sum())} positions selected, all equal")


def test_dsa_full_workload():
    prob = workloads.dsa_workload("dsa_decode")
    say(f"[gpu] dsa full workload: q{tuple(prob.query.shape)} k{tuple(prob.key.shape)} top_k {prob.top_k}")
    got, _ = _run(prob)
    want = dsa_oracle.index_select(prob.query, prob.key, prob.weights, prob.bias, **prob.kwargs())
    assert np.array_equal(got, want)


def test_dsa_small_workload_and_reuse():
    """The small workload, twice on one workspace (the second call overwrites the first's keys)."""
    prob = workloads.dsa_workload("dsa_decode", small=True)
    other = workloads.dsa_workload("dsa_decode", small=True, seed=99)
    B, S, _, _ = prob.query.shape
    T = prob.key.shape[1]
    ws = torch.empty(fa.dsa_workspace_bytes(B, S, T), dtype=torch.uint8, device="cuda")
    say("[gpu] dsa small workload, workspace reuse")
    a, _ = _run(other, ws)
    b, _ = _run(prob, ws)
    assert np.array_equal(a, dsa_oracle.index_select(other.query, other.key, other.weights, other.bias, **other.kwargs()))
    assert np.array_equal(b, dsa_oracle.index_select(prob.query, prob.key, prob.weights, prob.bias, **prob.kwargs()))


def test_dsa_no_heads_with_null_query_key_and_weights():
    """With no heads the scores are the bias alone; query, key and weights may be NULL."""
    prob = workloads.make_dsa_problem(seed=91, batch=1, q_seq=2, heads=0, head_dim=16, key_seq=300,
                                      top_k=10, dtype="bf16", bias="random")
    B, S, _, _ = prob.query.shape
    T = prob.key.shape[1]
    bias = prob.bias.to("cuda")
    out = torch.empty((B, 1, S, prob.top_k), dtype=torch.int64, device="cuda")
    ws = torch.empty(fa.dsa_workspace_bytes(B, S, T), dtype=torch.uint8, device="cuda")
    say("[gpu] dsa no heads, NULL query/key/weights")
    lib = fa._load()
    status = lib.dsa_index_select(None, None, None, bias.data_ptr(), out.data_ptr(), B, S, 0, 16, T,
                                  prob.top_k, prob.scale, prob.weights_scale, fa.FA_DTYPE_BF16,
                                  ws.data_ptr(), ws.numel(), torch.cuda.current_stream().cuda_stream)
    assert status == fa.FA_OK, fa.last_error()
    torch.cuda.synchronize()
    want = dsa_oracle.index_select(prob.query, prob.key, prob.weights, prob.bias, **prob.kwargs())
    assert np.array_equal(out.cpu().numpy(), want)


def test_dsa_no_keys_gives_minus_one():
    prob = workloads.make_dsa_problem(seed=89, batch=2, q_seq=3, heads=2, head_dim=8, key_seq=0,
                                      top_k=5, dtype="bf16")
    say("[gpu] dsa key_seq=0")
    got, _ = _run(prob)
    assert (got == -1).all()


def test_dsa_graph_replay():
    prob = workloads.make_dsa_problem(name="graph", **CASES["f16_chunk_padding"])
    d = prob.to("cuda")
    B, S, _, _ = prob.query.shape
    T = prob.key.shape[1]
    ws = torch.empty(fa.dsa_workspace_bytes(B, S, T), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, 1, S, prob.top_k), dtype=torch.int64, device="cuda")
    say("[gpu] dsa graph replay")
    fa.dsa_index_select(d.query, d.key, d.weights, d.bias, out=out, workspace=ws, **prob.kwargs())
    torch.cuda.synchronize()
    eager = out.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fa.dsa_index_select(d.query, d.key, d.weights, d.bias, out=out, workspace=ws, **prob.kwargs())
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(-9)
        ws.fill_(7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep}"
    want = dsa_oracle.index_select(prob.query, prob.key, prob.weights, prob.bias, **prob.kwargs())
    assert np.array_equal(out.cpu().numpy(), want)


def test_dsa_on_a_side_stream():
    """The call runs on the stream it is given; results read after that stream is synchronised."""
    prob = workloads.make_dsa_problem(name="side", **CASES["bf16_decode_d128"])
    d = prob.to("cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())   # inputs were copied on the default stream
    say("[gpu] dsa side stream")
    with torch.cuda.stream(side):
        out = fa.dsa_index_select(d.query, d.key, d.weights, d.bias, stream=side, **prob.kwargs())
    side.synchronize()
    want = dsa_oracle.index_select(prob.query, prob.key, prob.weights, prob.bias, **prob.kwargs())
    assert np.array_equal(out.cpu().numpy(), want)


def test_dsa_side_stream_not_current_keeps_workspace(monkeypatch):
    """stream= names a stream that is not the current one: the workspace the binding allocates
    must not be handed to work on the current stream before the side stream's kernels ran."""
    from gpu_util import AllocSpy, busy_stream, churn_hits

    prob = workloads.make_dsa_problem(name="side2", **CASES["bf16_decode_d128"])
    d = prob.to("cuda")
    B, S, _, _ = prob.query.shape
    need = fa.dsa_workspace_bytes(B, S, prob.key.shape[1])
    side = busy_stream()
    spy = AllocSpy()
    say("[gpu] dsa on a side stream that is not current, allocations churned meanwhile")
    monkeypatch.setattr(torch, "empty", spy)
    out = fa.dsa_index_select(d.query, d.key, d.weights, d.bias, stream=side, **prob.kwargs())
    monkeypatch.undo()
    assert spy.ptrs, "the binding allocated nothing"
    hits = churn_hits(spy.ptrs - {out.data_ptr()}, need)
    side.synchronize()
    assert hits == 0, "the workspace was reused while the side stream still needed it"
    want = dsa_oracle.index_select(prob.query, prob.key, prob.weights, prob.bias, **prob.kwargs())
    assert np.array_equal(out.cpu().numpy(), want)
