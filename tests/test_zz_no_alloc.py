"""flash_attn_fwd_splitkv_noalloc (the split-key path on the library's static device scratch)
against flash_attn_fwd_splitkv with a caller workspace, through the C ABI: two calls in a row on
one device, the second smaller, each bit-identical to the workspace call at the same span count
and within the 16-bit tolerance of the oracle."""

import pytest
import torch

import tiled_online_softmax_flash_amd as fa
import workloads
from gpu_util import check, oracle_full, say

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

CALLS = [
    # the decode workload's reduced copy: 3 sequences, 4 query heads per KV head, 1000 keys
    ("decode_b3", dict(workloads.SMALL_WORKLOADS["gqa_decode"], lengths="total",
                       nan_beyond_total=True), None),
    # smaller: one KV head, 2 query rows of 4 heads, f16 head dim 64, softcap, window, and a
    # per-batch float32 mask with -inf holes; fixed span count 8
    ("masked_b2", dict(seed=91, batch=2, heads=4, kv_heads=1, sq=2, sk=300, dim=64, dtype="f16",
                       causal=True, local_window=200, softcap=30.0, mask="bernoulli",
                       mask_p=0.2), 8),
]


def _outputs(prob, splits):
    d = prob.to("cuda")
    kw = d.kwargs()
    shape = (prob.batch, prob.heads, prob.sq, prob.dim) if prob.out_layout == "head" else (
        prob.batch, prob.sq, prob.heads * prob.dim)
    if splits is None:
        splits = fa.splitkv_suggested_splits(prob.batch, prob.kv_heads, prob.sk)
    need = fa.splitkv_workspace_bytes(prob.batch, prob.kv_heads, prob.dim, splits)
    assert 0 < need <= fa.SPLITKV_NOALLOC_SCRATCH_BYTES
    ref = torch.full(shape, float("nan"), dtype=prob.q.dtype, device="cuda")
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda")
    fa.flash_attn_fwd_splitkv(d.q, d.k, d.v, out=ref, num_splits=splits, workspace=ws, **kw)
    got = torch.full(shape, float("nan"), dtype=prob.q.dtype, device="cuda")
    fa.flash_attn_fwd_splitkv_noalloc(d.q, d.k, d.v, out=got, num_splits=splits, **kw)
    torch.cuda.synchronize()
    return got, ref, splits


def test_noalloc_matches_workspace_entry_point_twice():
    for name, params, splits in CALLS:
        prob = workloads.make_problem(name=name, **params)
        say(f"[gpu] noalloc {name}: q{tuple(prob.q.shape)} sk={prob.sk} {prob.dtype} splits={splits}")
        got, ref, used = _outputs(prob, splits)
        assert torch.equal(got, ref), f"{name}: static-scratch output differs from the workspace call"
        check(got.double().cpu().numpy(), oracle_full(prob), prob.dtype, f"noalloc-{name}-{used}")


def test_noalloc_rejects_state_beyond_the_scratch():
    q = torch.zeros(64, 8, 1, 128, dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros(64, 8, 4096, 128, dtype=torch.bfloat16, device="cuda")
    # 64 spans x 512 groups x 32 rows x 130 floats = 545 MB of state > 16 MiB
    with pytest.raises(fa.FaError) as err:
        fa.flash_attn_fwd_splitkv_noalloc(q, kv, kv, num_splits=64)
    assert err.value.status == fa.FA_ERR_UNSUPPORTED
