"""flash_attn_fwd captured into a HIP graph and replayed.

A call enqueues exactly one kernel on the caller's stream (none for an empty problem), with no
allocation, memset or synchronisation, so it can be captured once and replayed.  The graph
keeps the tensors' addresses: a replay reads whatever the buffers hold at that moment.  Each
replay here runs after eager work and a synchronisation, and is checked against an eager call
on the same inputs (bit for bit) and against the oracle.
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
    # 256-row kernel: GQA, causal, ragged last query tile
    "bf16_gqa_causal": dict(seed=60, batch=2, heads=8, kv_heads=2, sq=300, sk=300, dim=128,
                            dtype="bf16", causal=True),
    # 256-row kernel with an additive mask and device-side lengths
    "bf16_mask_lengths": dict(seed=61, batch=2, heads=4, kv_heads=2, sq=130, sk=260, dim=64,
                              dtype="bf16", mask="bernoulli", mask_p=0.1, causal=True,
                              lengths="past", max_past=100),
    # fp32 kernel, token-major output
    "f32_token_major": dict(seed=62, batch=1, heads=3, kv_heads=1, sq=100, sk=120, dim=128,
                            dtype="f32", out_layout="token"),
}


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replay_matches_eager(name):
    prob = workloads.make_problem(name=name, **CASES[name])
    other = workloads.make_problem(name=name + "_b", **dict(CASES[name], seed=CASES[name]["seed"] + 100))
    say(f"[gpu] graph {name}: q{tuple(prob.q.shape)} {prob.dtype}")
    d = prob.to("cuda")
    d2 = other.to("cuda")
    kw = d.kwargs()
    out = fa.flash_attn_fwd(d.q, d.k, d.v, **kw)   # eager call before capture
    torch.cuda.synchronize()
    eager = out.clone()
    eager2 = fa.flash_attn_fwd(d2.q, d.k, d.v, **kw).clone()   # other queries, same keys
    torch.cuda.synchronize()

    q_saved = d.q.clone()
    graph = torch.cuda.CUDAGraph()
    out.fill_(float("nan"))
    with torch.cuda.graph(graph):
        fa.flash_attn_fwd(d.q, d.k, d.v, out=out, **kw)
    torch.cuda.synchronize()

    for rep in range(4):
        use_other = rep % 2 == 1
        # eager work between replays: refill the output, swap the queries in place
        out.fill_(float("nan"))
        d.q.copy_(d2.q if use_other else q_saved)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        want = eager2 if use_other else eager
        assert torch.equal(out, want), f"{name}: replay {rep} differs from the eager call"
    d.q.copy_(q_saved)
    graph.replay()
    torch.cuda.synchronize()
    check(out.double().cpu().numpy(), oracle_full(prob), prob.dtype, f"graph-{name}")
