"""Helpers for the GPU parity tests: run the HIP path through the C ABI and compare with the
oracle on the same seeded inputs."""

from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import tiled_online_softmax_flash_amd as fa

# max-abs tolerances of the output vs the f64 oracle
TOL = {"f32": 1e-4, "f16": 2e-2, "bf16": 2e-2}


def say(msg: str) -> None:
    """Name the GPU step about to run, unbuffered (survives a lost box)."""
    print(msg, file=sys.__stderr__, flush=True)


def misaligned_copy(t: torch.Tensor) -> torch.Tensor:
    """A contiguous device copy of ``t`` whose data starts one element past a 256-byte boundary
    (2 bytes for 16-bit types, 4 for float32), so no row starts on a 16-byte boundary."""
    buf = torch.empty(t.numel() + 1, dtype=t.dtype, device="cuda")
    view = buf[1:].view(t.shape)
    view.copy_(t)
    assert view.is_contiguous() and view.data_ptr() % 16 != 0
    return view


def run_gpu(prob, out_fill: float | None = None, splitkv: bool = False,
            misalign: bool = False) -> torch.Tensor:
    """The problem on cuda:0 through flash_attn_fwd (or flash_attn_fwd_splitkv with the device's
    suggested number of spans); returns the output on the GPU.  ``misalign`` passes q, k, v and
    out at addresses one element off 16-byte alignment (contiguous all the same)."""
    d = prob.to("cuda")
    shape = (prob.batch, prob.heads, prob.sq, prob.dim) if prob.out_layout == "head" else (
        prob.batch, prob.sq, prob.heads * prob.dim)
    out = None
    if out_fill is not None or misalign:
        out = torch.full(shape, float("nan") if out_fill is None else out_fill, dtype=prob.q.dtype,
                         device="cuda")
    if misalign:
        d.q, d.k, d.v, out = (misaligned_copy(t) for t in (d.q, d.k, d.v, out))
    kw = d.kwargs()
    if splitkv:
        res = fa.flash_attn_fwd_splitkv(d.q, d.k, d.v, out=out, **kw)
    else:
        res = fa.flash_attn_fwd(d.q, d.k, d.v, out=out, **kw)
    torch.cuda.synchronize()
    return res


def oracle_full(prob) -> np.ndarray:
    return oracle.forward(prob.q, prob.k, prob.v, **prob.kwargs())


def oracle_rows(prob, rows) -> np.ndarray:
    return oracle.rows(prob.q, prob.k, prob.v, rows, **prob.kwargs())


def gpu_rows(out: torch.Tensor, prob, rows) -> np.ndarray:
    """Rows (b, h, i) of a GPU output in either layout, as float64 [n, D]."""
    D = prob.dim
    host = out.double().cpu().numpy()
    res = np.empty((len(rows), D))
    for n, (b, h, i) in enumerate(rows):
        if prob.out_layout == "head":
            res[n] = host[b, h, i]
        else:
            res[n] = host[b, i, h * D:(h + 1) * D]
    return res


def check(got: np.ndarray, want: np.ndarray, dtype: str, name: str, amp: float = 1.0) -> dict:
    """Max-abs gate at the dtype's tolerance, scaled by the input amplitude ``amp`` (>= 1).

    With fp32 accumulation the 16-bit paths' error comes from rounding the weights P to the
    input type before the P.V product and from rounding the output.  An output row is a convex
    combination of V rows, so both errors are at most a small multiple of the unit roundoff times
    max |v|; the scores' own fp32 error is far smaller.  Inputs scaled by ``amp`` scale max |v|
    by ``amp`` (the weights stay in [0, 1]), so the error bound, and the gate, scale linearly
    with ``amp``."""
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    err = np.abs(got - want)
    max_abs = float(err.max()) if err.size else 0.0
    rel = float((err / np.maximum(np.abs(want), 1e-2)).max()) if err.size else 0.0
    tol = TOL[dtype] * max(amp, 1.0)
    say(f"  {name}: max_abs={max_abs:.3e} max_rel(floor 1e-2)={rel:.3e} tol={tol:.0e}")
    assert max_abs <= tol, f"{name}: max abs error {max_abs:.3e} > {tol:.0e}"
    # rows the oracle returns as exactly zero (nothing attended) must be exactly zero
    zero_rows = np.all(want == 0.0, axis=-1)
    if zero_rows.any():
        assert np.all(got[zero_rows] == 0.0), f"{name}: fully masked rows are not exactly 0"
    return dict(max_abs=max_abs, max_rel=rel)


def sample_rows(prob, n: int, seed: int = 1234, extra=()) -> list:
    rng = np.random.Generator(np.random.PCG64(seed))
    rows = set(tuple(int(x) for x in r) for r in extra)
    B, H, Sq = prob.batch, prob.heads, prob.sq
    for corner in [(0, 0, 0), (B - 1, H - 1, Sq - 1), (0, H - 1, Sq // 2), (B - 1, 0, Sq - 1)]:
        rows.add(corner)
    target = min(B * H * Sq, n + len(rows))
    while len(rows) < target:
        rows.add((int(rng.integers(B)), int(rng.integers(H)), int(rng.integers(Sq))))
    return sorted(rows)


def busy_stream(seconds_hint: int = 30) -> torch.cuda.Stream:
    """A new stream held busy by a chain of fp32 matrix products (tens of milliseconds), after
    waiting for the current stream's work (the inputs' copies)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        a = torch.full((2048, 2048), 1e-3, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(seconds_hint):
            torch.mm(a, a, out=b)
            torch.mm(b, b, out=a)
    return side


class AllocSpy:
    """Records the tensors torch.empty returns while installed (monkeypatched by a test)."""

    def __init__(self):
        self.ptrs = set()
        self._real = torch.empty

    def __call__(self, *args, **kwargs):
        t = self._real(*args, **kwargs)
        if t.is_cuda and t.numel():
            self.ptrs.add(t.data_ptr())
        return t


def churn_hits(ptrs, nbytes: int, rounds: int = 64) -> int:
    """Allocates and fills ``rounds`` byte tensors of ``nbytes`` on the current stream; returns how
    many of them landed on an address in ``ptrs``."""
    hits = 0
    for _ in range(rounds):
        y = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
        hits += int(y.data_ptr() in ptrs)
        y.fill_(0xFF)
        del y
    return hits
