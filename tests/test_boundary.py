"""The C-ABI library on the CPU: it loads, exports every declared entry point, and validates
arguments (no kernel is launched; validation touches no HIP state)."""

import ctypes
import os
import re

import pytest
import torch

import tiled_online_softmax_flash_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    assert declared_functions() == ["fa_check_args", "fa_last_error", "fa_splitkv_suggested_splits",
                                    "fa_splitkv_workspace_bytes", "fa_version", "flash_attn_fwd",
                                    "flash_attn_fwd_splitkv", "flash_attn_fwd_splitkv_noalloc"]


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(fa.library_path)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version():
    assert fa.version() == "0.1.0"


GOOD = dict(q=16, k=16, v=16, out=16, batch=2, heads=8, kv_heads=2, sq=100, sk=90,
            kv_capacity=128, dim=64, causal=1, mask_planes=0, local_window=0, scale=0.125,
            softcap=0.0, dtype=fa.FA_DTYPE_BF16, mask_dtype=fa.FA_DTYPE_F32, out_layout=0)


def status(**over):
    args = dict(GOOD)
    args.update(over)
    return fa.check_args(**args)


def test_valid_arguments_pass():
    assert status() == fa.FA_OK
    assert status(dtype=fa.FA_DTYPE_F32) == fa.FA_OK
    assert status(dtype=fa.FA_DTYPE_F16, out_layout=1) == fa.FA_OK
    assert status(mask=16, mask_planes=2) == fa.FA_OK
    assert status(mask=16, mask_planes=16, mask_dtype=fa.FA_DTYPE_BF16) == fa.FA_OK
    assert status(mask=16, mask_planes=1) == fa.FA_OK
    for d in (1, 7, 40, 80, 128):
        assert status(dim=d) == fa.FA_OK, d
    for d in (129, 200, 384):   # fp32 goes up to 384
        assert status(dim=d, dtype=fa.FA_DTYPE_F32) == fa.FA_OK, d
    assert status(softcap=50.0, local_window=1024) == fa.FA_OK
    assert status(scale=0.0) == fa.FA_OK and status(scale=-1.0) == fa.FA_OK


@pytest.mark.parametrize("over,code", [
    (dict(dtype=3), fa.FA_ERR_UNSUPPORTED),
    (dict(dim=0), fa.FA_ERR_UNSUPPORTED),
    (dict(dim=129), fa.FA_ERR_UNSUPPORTED),
    (dict(dim=129, dtype=fa.FA_DTYPE_F16), fa.FA_ERR_UNSUPPORTED),
    (dict(dim=385, dtype=fa.FA_DTYPE_F32), fa.FA_ERR_UNSUPPORTED),
    (dict(mask=16, mask_planes=2, mask_dtype=fa.FA_DTYPE_F16), fa.FA_ERR_UNSUPPORTED),
    (dict(out_layout=2), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(batch=-1), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(sq=-5), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(kv_heads=0), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(heads=6, kv_heads=4), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(sk=129), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(mask=16, mask_planes=3), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(mask=None, mask_planes=2), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(mask=16, mask_planes=-2), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(scale=float("inf")), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(softcap=float("nan")), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(q=None), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(out=None), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(k=None), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(batch=2**30, heads=2**30, kv_heads=1), fa.FA_ERR_OVERFLOW),
    (dict(batch=2**20, heads=2**16, kv_heads=1, sq=2**20, kv_capacity=1, sk=1, dim=128),
     fa.FA_ERR_OVERFLOW),
    (dict(mask=16, mask_planes=2**20, batch=2**20, heads=1, kv_heads=1, sq=2**20, sk=2**20,
          kv_capacity=2**20), fa.FA_ERR_OVERFLOW),
    (dict(batch=2**16, heads=2**16, kv_heads=1, sq=1, dim=1), fa.FA_ERR_OVERFLOW),
])
def test_invalid_arguments_are_rejected(over, code):
    assert status(**over) == code
    assert fa.last_error() != ""


def test_empty_problems_are_ok_without_pointers():
    assert status(batch=0, q=None, k=None, v=None, out=None) == fa.FA_OK
    assert status(sq=0, q=None, out=None) == fa.FA_OK
    assert status(heads=0, q=None, out=None) == fa.FA_OK
    # no keys at all: k and v may be null, the rows are written as zeros
    assert status(sk=0, kv_capacity=0, k=None, v=None) == fa.FA_OK


def test_binding_rejects_host_tensors():
    q = torch.zeros(1, 1, 4, 8, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.flash_attn_fwd(q, q, q)


def test_binding_rejects_mismatched_shapes_and_dtypes():
    q = torch.zeros(1, 2, 4, 8)
    with pytest.raises(ValueError):
        fa.flash_attn_fwd(q, torch.zeros(1, 2, 4, 16), torch.zeros(1, 2, 4, 16))
    with pytest.raises(ValueError):
        fa.flash_attn_fwd(q, q.double(), q.double())


# ---- split-key (decode) entry point: its own checks, all taken before any launch

def splitkv_status(num_splits=8, workspace=16, workspace_bytes=None, **over):
    """flash_attn_fwd_splitkv's status for fake device pointers (no check dereferences them)."""
    args = dict(GOOD, sq=1, heads=8, kv_heads=2, dim=128)
    args.update(over)
    if workspace_bytes is None:
        workspace_bytes = fa.splitkv_workspace_bytes(args["batch"], args["kv_heads"], args["dim"], num_splits)
    fa._load()   # sets the argument types
    f = fa._lib.flash_attn_fwd_splitkv
    return f(args["q"], args["k"], args["v"], args.get("mask"), None, None, args["out"], args["batch"],
             args["heads"], args["kv_heads"], args["sq"], args["sk"], args["kv_capacity"], args["dim"],
             args["causal"], args["mask_planes"], args["local_window"], args["scale"], args["softcap"],
             args["dtype"], args["mask_dtype"], args["out_layout"], num_splits, workspace,
             workspace_bytes, None)


def test_splitkv_workspace_bytes():
    assert fa.splitkv_workspace_bytes(8, 8, 128, 16) == 16 * 8 * 8 * 32 * 130 * 4
    assert fa.splitkv_workspace_bytes(1, 1, 64, 4) == 4 * 32 * 66 * 4
    assert fa.splitkv_workspace_bytes(1, 1, 64, 0) == 0
    assert fa.splitkv_workspace_bytes(2**30, 2**30, 128, 4) == 0   # overflow


@pytest.mark.parametrize("over,code", [
    (dict(dtype=fa.FA_DTYPE_F32), fa.FA_ERR_UNSUPPORTED),
    (dict(dim=96), fa.FA_ERR_UNSUPPORTED),
    (dict(sq=9), fa.FA_ERR_UNSUPPORTED),                       # 4 heads per KV head x 9 rows > 32
    (dict(q=8), fa.FA_ERR_UNSUPPORTED),                        # misaligned
    (dict(num_splits=6), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(num_splits=0), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(workspace=None), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(workspace=24), fa.FA_ERR_INVALID_ARGUMENT),          # misaligned workspace
    (dict(workspace_bytes=1024), fa.FA_ERR_INVALID_ARGUMENT),  # too small
    (dict(heads=6, kv_heads=4), fa.FA_ERR_INVALID_ARGUMENT),   # shared check
])
def test_splitkv_rejects(over, code):
    assert splitkv_status(**over) == code, fa.last_error()


def test_splitkv_takes_masks():
    # sq = 0: every check runs, then the empty problem returns before any launch
    assert splitkv_status(mask=16, mask_planes=2, sq=0) == fa.FA_OK
    assert splitkv_status(mask=16, mask_planes=16, mask_dtype=fa.FA_DTYPE_BF16, sq=0) == fa.FA_OK
    assert splitkv_status(mask=None, mask_planes=2) == fa.FA_ERR_INVALID_ARGUMENT


def test_splitkv_empty_problem_is_a_no_op():
    assert splitkv_status(sq=0) == fa.FA_OK


def noalloc_status(num_splits=8, **over):
    """flash_attn_fwd_splitkv_noalloc's status for fake device pointers."""
    args = dict(GOOD, sq=1, heads=8, kv_heads=2, dim=128)
    args.update(over)
    fa._load()
    f = fa._lib.flash_attn_fwd_splitkv_noalloc
    return f(args["q"], args["k"], args["v"], args.get("mask"), None, None, args["out"], args["batch"],
             args["heads"], args["kv_heads"], args["sq"], args["sk"], args["kv_capacity"], args["dim"],
             args["causal"], args["mask_planes"], args["local_window"], args["scale"], args["softcap"],
             args["dtype"], args["mask_dtype"], args["out_layout"], num_splits, None)


def test_noalloc_checks_before_touching_the_device():
    # every check of the workspace entry point except the workspace's own, then the scratch limit;
    # all of them return before the scratch's address is looked up
    assert noalloc_status(sq=0) == fa.FA_OK
    assert noalloc_status(dtype=fa.FA_DTYPE_F32) == fa.FA_ERR_UNSUPPORTED
    assert noalloc_status(num_splits=6) == fa.FA_ERR_INVALID_ARGUMENT
    assert noalloc_status(heads=6, kv_heads=4) == fa.FA_ERR_INVALID_ARGUMENT
    # 64 batch x 8 KV heads x 64 spans x 32 rows x 130 floats = 545 MB > the 16 MiB scratch
    need = fa.splitkv_workspace_bytes(64, 8, 128, 64)
    assert need > fa.SPLITKV_NOALLOC_SCRATCH_BYTES
    assert noalloc_status(batch=64, heads=32, kv_heads=8, sk=4096, kv_capacity=4096,
                          num_splits=64) == fa.FA_ERR_UNSUPPORTED
    assert "static scratch" in fa.last_error()


def test_noalloc_scratch_size_matches_the_header():
    text = open(HEADER).read()
    m = re.search(r"#define FA_SPLITKV_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == fa.SPLITKV_NOALLOC_SCRATCH_BYTES


# ---- sparse index selection (include/dsa.h)

DSA_HEADER = os.path.join(ROOT, "include", "dsa.h")


def test_dsa_header_declares_its_functions_and_the_library_exports_them():
    text = re.sub(r"/\*.*?\*/", "", open(DSA_HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", text, flags=re.M)))
    assert names == ["dsa_check_args", "dsa_index_select", "dsa_index_select_workspace_bytes"]
    lib = ctypes.CDLL(fa.library_path)
    for name in names:
        assert hasattr(lib, name), name


DSA_GOOD = dict(query=16, key=16, weights=16, bias=16, out=16, batch=2, q_seq=3, heads=4,
                head_dim=64, key_seq=1000, top_k=64, scale=0.125, weights_scale=1.0,
                dtype=fa.FA_DTYPE_BF16, workspace=256, workspace_bytes=None)


def dsa_status(**over):
    a = dict(DSA_GOOD)
    a.update(over)
    if a["workspace_bytes"] is None:
        a["workspace_bytes"] = fa.dsa_workspace_bytes(a["batch"], a["q_seq"], a["key_seq"])
    return fa.dsa_check_args(a["query"], a["key"], a["weights"], a["bias"], a["out"], a["batch"],
                             a["q_seq"], a["heads"], a["head_dim"], a["key_seq"], a["top_k"],
                             a["scale"], a["weights_scale"], a["dtype"], a["workspace"],
                             a["workspace_bytes"])


def test_dsa_workspace_bytes():
    # keys (4 B per cell), then per row 4104 words and one word per 2048-position chunk, then
    # 8 B per cell (candidates)
    assert fa.dsa_workspace_bytes(2, 3, 1000) == 2 * 3 * 1000 * 12 + 6 * 4104 * 4 + 6 * 1 * 4
    assert fa.dsa_workspace_bytes(1, 2, 4097) == 2 * 4097 * 12 + 2 * 4104 * 4 + 2 * 3 * 4
    assert fa.dsa_workspace_bytes(2, 3, 0) == 0
    assert fa.dsa_workspace_bytes(-1, 3, 10) == 0
    assert fa.dsa_workspace_bytes(2**30, 2**30, 2**30) == 0


def test_dsa_valid_arguments_pass():
    assert dsa_status() == fa.FA_OK
    for dt in (fa.FA_DTYPE_F32, fa.FA_DTYPE_F16):
        assert dsa_status(dtype=dt) == fa.FA_OK
    for d in (0, 1, 33, 100, 128):
        assert dsa_status(head_dim=d) == fa.FA_OK, d
    assert dsa_status(top_k=5000) == fa.FA_OK          # wider than the key range: -1 padding
    assert dsa_status(heads=0, query=None, weights=None) == fa.FA_OK
    assert dsa_status(heads=0, query=None, key=None, weights=None) == fa.FA_OK   # scores = bias
    assert dsa_status(batch=0, query=None, key=None, weights=None, bias=None, out=None, workspace=None) == fa.FA_OK
    assert dsa_status(key_seq=0, key=None, bias=None, workspace=None) == fa.FA_OK


@pytest.mark.parametrize("over,code", [
    (dict(dtype=3), fa.FA_ERR_UNSUPPORTED),
    (dict(head_dim=129), fa.FA_ERR_UNSUPPORTED),
    (dict(top_k=0), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(scale=0.0), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(scale=float("inf")), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(weights_scale=-1.0), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(weights_scale=float("nan")), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(batch=-1), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(key_seq=-3), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(out=None), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(out=12), fa.FA_ERR_INVALID_ARGUMENT),         # int64 output not 8-byte aligned
    (dict(bias=None), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(query=None), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(weights=None), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(workspace=None), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(workspace=264), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(workspace_bytes=100), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(batch=2**16, q_seq=2**16, key_seq=2**16), fa.FA_ERR_OVERFLOW),
    (dict(batch=2**20, q_seq=2**11, key_seq=2**20, top_k=1, workspace_bytes=2**62), fa.FA_ERR_OVERFLOW),
])
def test_dsa_invalid_arguments_are_rejected(over, code):
    assert dsa_status(**over) == code, fa.last_error()
    assert fa.last_error() != ""


def test_new_bindings_reject_host_tensors():
    q = torch.zeros(1, 4, 1, 64, dtype=torch.bfloat16)
    k = torch.zeros(1, 1, 32, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.flash_attn_fwd_splitkv(q, k, k)
    with pytest.raises(ValueError):
        fa.dsa_index_select(torch.zeros(1, 1, 2, 8), torch.zeros(1, 5, 8), torch.zeros(1, 1, 2),
                            torch.zeros(1, 1, 1, 5), top_k=2, scale=1.0)


def test_dsa_binding_checks_shapes_and_dtypes():
    q, k, w, b = torch.zeros(1, 1, 2, 8), torch.zeros(1, 5, 8), torch.zeros(1, 1, 2), torch.zeros(1, 1, 1, 5)
    with pytest.raises(ValueError):
        fa.dsa_index_select(q, torch.zeros(1, 5, 4), w, b, top_k=2, scale=1.0)      # head dim
    with pytest.raises(ValueError):
        fa.dsa_index_select(q, k, w, b.double(), top_k=2, scale=1.0)               # bias dtype
    with pytest.raises(ValueError):
        fa.dsa_index_select(q, k.half(), w, b, top_k=2, scale=1.0)                 # mixed dtypes


def test_bench_refuses_more_than_one_gpu(capsys):
    import bench

    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err
