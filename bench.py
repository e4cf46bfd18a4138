"""Benchmark of the MI355X tiled online-softmax attention forward.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload gqa_causal] [--no-cpu-baseline]

One step = one flash_attn_fwd launch over the whole workload (inputs resident in HBM).  Prints
one JSON line: attention-forward TFLOP/s (4*B*H*Sq*Sk_eff*D per step over the wall time of K
steps), the dominant kernel's roofline (its average duration: HIP events recorded on the launch
stream before the first and after the last of the K back-to-back timed launches, divided by K)
and the f64 oracle timed on a bounded sample of the same workload on the host cores.

The decode workload (gqa_decode) runs through flash_attn_fwd_splitkv instead: one step is its
two kernels (spans, then merge), and the roofline is HBM-bound: the step's algorithmic bytes
(Q, the attended K/V rows, O) over the event time of the two kernels, against 8 TB/s.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import tiled_online_softmax_flash_amd as fa  # noqa: E402
import workloads  # noqa: E402
from tiled_online_softmax_flash_amd.metrics import attended_counts, problem_work  # noqa: E402

# MI355X published dense peaks (TFLOP/s) and HBM bandwidth (GB/s)
PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "f32": 157.3}
PEAK_HBM_GBS = 8000.0
# Exponentials per second: the fp32 vector peak of 157.3 TFLOP/s counts a packed fused
# multiply-add (2 lanes x 2 flops) per lane slot, i.e. 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz
# = 39.3 T plain lane operations per second; transcendental instructions (v_exp_f32) issue at
# half that rate on gfx950 (a microbenchmark of independent v_exp_f32 chains measures 3.2 plain
# multiply-adds' worth of time each, at the box's own clock).  The softmax takes one exponential
# per attended score, the secondary ceiling the attention kernels are held to.
PEAK_EXP_PER_S = 256 * 4 * 16 * 2.4e9 / 2
METRIC = "attention fwd TFLOP/s (4·B·H·Sq·Sk_eff·D) + % of MI355X MFMA peak"
KERNEL_SOURCES = ["fa_device.h", "fa_params.h", "fa_fwd16.h", "fa_fwd16_ring.h",
                  "fa_fwd16_ring_consts.h", "fa_fwd32.h", "fa_fwd32w.h", "fa_splitkv.h",
                  "fa_launch.h", "fa_api.hip", "dsa_select.hip", "dsa_kernels.h"]


def kernel_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "tiled_online_softmax_flash_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profile(workload: str):
    """HBM bytes per launch from committed counter runs, if taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_hash") != kernel_hash():
        return None
    return rec.get("traffic_bytes")


def warm_up(step, count: int, min_seconds: float) -> float:
    """Runs ``count`` untimed steps, then keeps running steps until at least ``min_seconds`` of
    wall time have passed since the first one; returns the seconds spent.

    The GPU's clocks ramp up over the first few tenths of a second of sustained load (from idle,
    the first launches of the GQA causal workload run 15-30 % slower), so a warm-up given only
    as a step count can leave a short timed region measuring the ramp instead of the kernel."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(count):
        step()
    torch.cuda.synchronize()
    batch = 8
    while time.perf_counter() - t0 < min_seconds:
        for _ in range(batch):
            step()
        torch.cuda.synchronize()
        batch = min(batch * 2, 256)
    return time.perf_counter() - t0


def cpu_baseline(prob, out_gpu: torch.Tensor, target_s: float):
    """The oracle as it stands, timed on a bounded row sample of the same workload."""
    import oracle

    orc = oracle.default()
    threads = orc.default_threads()
    counts = attended_counts(prob.batch, prob.sq, prob.sk, prob.causal, prob.local_window,
                             None if prob.total_lengths is None else prob.total_lengths.numpy(),
                             None if prob.past_lengths is None else prob.past_lengths.numpy())
    rng = np.random.Generator(np.random.PCG64(99))

    def pick(n):
        return [(int(rng.integers(prob.batch)), int(rng.integers(prob.heads)),
                 int(rng.integers(prob.sq))) for _ in range(n)]

    # calibrate on growing samples until one takes >= 0.5 s, then size the timed sample to
    # about target_s seconds of oracle work
    n_cal = max(threads * 4, 32)
    while True:
        calib = pick(n_cal)
        t0 = time.perf_counter()
        orc.rows(prob.q, prob.k, prob.v, calib, **prob.kwargs())
        dt = time.perf_counter() - t0
        if dt >= 0.5 or n_cal >= prob.batch * prob.heads * prob.sq:
            break
        n_cal *= 4
    n = int(min(max(n_cal * target_s / max(dt, 1e-3), n_cal), prob.batch * prob.heads * prob.sq))
    rows = pick(n)
    t0 = time.perf_counter()
    want = orc.rows(prob.q, prob.k, prob.v, rows, **prob.kwargs())
    dt = time.perf_counter() - t0
    flops = 4.0 * prob.dim * float(sum(counts[b, i] for b, _, i in rows))
    host = out_gpu.double().cpu().numpy()
    D = prob.dim
    got = np.stack([host[b, h, i] if prob.out_layout == "head" else host[b, i, h * D:(h + 1) * D]
                    for b, h, i in rows])
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{n} random (b,h,i) output rows of the same workload, f64, {dt:.1f} s",
        "sample_max_abs_err_vs_gpu": float(np.abs(got - want).max()),
    }


# fp32 VALU lane operations per second: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz.  The scoring
# multiplies and adds are separate instructions (the operation fixes un-fused rounding), one
# float operation per lane each; the 157.3 TFLOP/s vector peak counts a packed fused multiply-add
# as four.
PEAK_VALU_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12


def bench_dsa(args) -> int:
    """The index-selection workload: one step = one dsa_index_select call (scoring + selection)."""
    prob = workloads.dsa_workload(args.workload)
    B, S, H, D = prob.query.shape
    T = prob.key.shape[1]
    d = prob.to("cuda")
    allowed = int((prob.bias > -1e30).sum())
    ops = 2 * H * D * allowed   # one multiply and one add per (allowed cell, head, dim)
    out = torch.empty((B, 1, S, prob.top_k), dtype=torch.int64, device="cuda")
    ws = torch.empty(max(fa.dsa_workspace_bytes(B, S, T), 1), dtype=torch.uint8, device="cuda")

    def step():
        fa.dsa_index_select(d.query, d.key, d.weights, d.bias, out=out, workspace=ws, **prob.kwargs())

    warm_s = warm_up(step, args.warmup, args.clock_warmup)
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    step_ms = ev0.elapsed_time(ev1) / args.steps
    result = {
        "metric": "DSA index selection: float32 score operations per second (2*H*D per allowed cell)",
        "value": round(ops / (ms_per_step * 1e-3) / 1e12, 3),
        "unit": "Tops/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "clock_warmup_s": round(warm_s, 3),
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": prob.dtype,
        "data": "synthetic (seeded N(0,1) query/key/weights, causal float32 bias)",
        "config": {"workload": args.workload, "batch": B, "q_seq": S, "heads": H, "head_dim": D,
                   "key_seq": T, "top_k": prob.top_k, "allowed_cells": allowed,
                   "entry_point": "dsa_index_select"},
        "roofline": {
            # event time of the whole step (scoring and selection kernels); the rocprofv3 summary
            # gives each kernel's share
            "bound": "alu",
            "achieved": round(ops / (step_ms * 1e-3) / 1e12, 3),
            "peak": round(PEAK_VALU_TOPS, 2),
            "unit": "Tops/s",
            "frac": round(ops / (step_ms * 1e-3) / 1e12 / PEAK_VALU_TOPS, 4),
            "traffic": None,
            "kernel_avg_us": round(step_ms * 1e3, 2),
            "algorithmic_ops_per_launch": ops,
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        from oracle import dsa as dsa_oracle

        host = out.cpu().numpy()
        rows, t_used = 0, 0.0
        t0 = time.perf_counter()
        # whole query rows of the workload, one after another, until about --cpu-seconds
        while rows < B * S and t_used < args.cpu_seconds:
            b, s_ = divmod(rows, S)
            sl = slice(s_, s_ + 1)
            got = dsa_oracle.index_select(prob.query[b:b + 1, sl], prob.key[b:b + 1],
                                          prob.weights[b:b + 1, sl], prob.bias[b:b + 1, :, sl],
                                          **prob.kwargs())
            assert np.array_equal(got[0, 0, 0], host[b, 0, s_]), "oracle and GPU disagree"
            rows += 1
            t_used = time.perf_counter() - t0
        row_ops = 2 * H * D * float((prob.bias[:, 0].reshape(B * S, T)[:rows] > -1e30).sum())
        result["cpu_baseline"] = {
            "value": row_ops / t_used / 1e12, "unit": "Tops/s", "cores": 1, "kind": "oracle",
            "sample": f"{rows} of {B * S} query rows of the same workload, scored and selected "
                      f"single-threaded in {t_used:.1f} s, every one equal to the GPU's",
        }
    print(json.dumps(result), flush=True)
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    # untimed steps continue after --warmup until this much wall time has passed: the GPU ramps
    # its clocks over the first ~0.1-0.3 s of sustained load, whatever the step count
    ap.add_argument("--clock-warmup", type=float, default=1.0, metavar="SECONDS")
    ap.add_argument("--workload", default="gqa_causal",
                    choices=list(workloads.WORKLOADS) + list(workloads.DSA_WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="instead of attention, run --steps plain device copies of BYTES bytes "
                         "(reference for scaling FETCH_SIZE/WRITE_SIZE counters)")
    ap.add_argument("--stream-reference", type=int, default=0, metavar="BYTES",
                    help="instead of attention, time a plain device copy and a read-only sum of "
                         "BYTES bytes (the streaming rates a bandwidth-bound kernel compares with)")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the op shards without "
              "communication over (batch, KV-head) groups, each GPU taking its own groups", file=sys.stderr)
        return 2
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2

    if args.stream_reference:
        n = args.stream_reference // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        res = {"bytes": 4 * n, "launches": args.steps}
        for name, fn, moved in (("copy", lambda: dst.copy_(src), 8 * n), ("sum", lambda: src.sum(), 4 * n)):
            for _ in range(20):
                fn()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(args.steps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / args.steps
            res[name] = {"us": round(us, 2), "gbs": round(moved / us / 1e3, 1),
                         "moved_bytes": moved}
        print(json.dumps(res), flush=True)
        return 0

    if args.copy_calibration:
        n = args.copy_calibration // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": 4 * n, "copy_bytes_written": 4 * n,
                          "launches": args.steps}), flush=True)
        return 0

    if args.workload in workloads.DSA_WORKLOADS:
        return bench_dsa(args)

    prob = workloads.workload(args.workload)
    work = problem_work(prob)
    dev = prob.to("cuda")
    out = torch.empty((prob.batch, prob.heads, prob.sq, prob.dim) if prob.out_layout == "head"
                      else (prob.batch, prob.sq, prob.heads * prob.dim), dtype=prob.q.dtype,
                      device="cuda")
    kw = dev.kwargs()
    splitkv = args.workload in workloads.SPLITKV_WORKLOADS
    if splitkv:
        # decode: the split-key entry point with a workspace allocated once, outside the loop
        splits = fa.splitkv_suggested_splits(prob.batch, prob.kv_heads, prob.sk)
        ws = torch.empty(fa.splitkv_workspace_bytes(prob.batch, prob.kv_heads, prob.dim, splits),
                         dtype=torch.uint8, device="cuda")

        def step():
            fa.flash_attn_fwd_splitkv(dev.q, dev.k, dev.v, out=out, num_splits=splits,
                                      workspace=ws, **kw)
    else:
        def step():
            fa.flash_attn_fwd(dev.q, dev.k, dev.v, out=out, **kw)

    warm_s = warm_up(step, args.warmup, args.clock_warmup)

    # one event pair around the whole timed region: per-launch event pairs would add their own
    # marker packets between the kernels
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    ms_per_step = wall * 1e3 / args.steps
    value = work["flops"] / (ms_per_step * 1e-3) / 1e12
    kern_avg_ms = ev0.elapsed_time(ev1) / args.steps
    if splitkv:
        # HBM-bound: the step's algorithmic bytes over the event time of its two kernels
        bound, unit, peak = "hbm", "GB/s", PEAK_HBM_GBS
        achieved = work["bytes"] / (kern_avg_ms * 1e-3) / 1e9
    else:
        bound, unit, peak = "mfma", "TFLOP/s", PEAK_TFLOPS[prob.dtype]
        achieved = work["flops"] / (kern_avg_ms * 1e-3) / 1e12
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_warmup_s": round(warm_s, 3),
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": prob.dtype,
        "data": "synthetic (seeded N(0,1) inputs of the workload's shape)",
        "config": {
            "workload": args.workload,
            "batch": prob.batch, "q_heads": prob.heads, "kv_heads": prob.kv_heads,
            "sq": prob.sq, "sk": prob.sk, "kv_capacity": prob.kv_capacity, "head_dim": prob.dim,
            "causal": prob.causal, "local_window": prob.local_window, "softcap": prob.softcap,
            "mask": None if prob.mask is None else list(prob.mask.shape),
            "out_layout": prob.out_layout, "sk_eff": round(work["sk_eff"], 3),
            "entry_point": "flash_attn_fwd_splitkv" if splitkv else "flash_attn_fwd",
            "global_batch": prob.batch, "seq_len": prob.sq, "parallelism": "none (1 GPU)",
        },
        "pct_of_peak": round(100.0 * value / PEAK_TFLOPS[prob.dtype], 2),
        "roofline": {
            "bound": bound,
            "achieved": round(achieved, 2),
            "peak": peak,
            "unit": unit,
            "frac": round(achieved / peak, 4),
            "traffic": traffic_from_profile(args.workload),
            "kernel_avg_us": round(kern_avg_ms * 1e3, 2),
            "algorithmic_flops_per_launch": work["flops"],
            "algorithmic_bytes_per_launch": work["bytes"],
            "hbm_gbs_at_algorithmic_bytes": round(work["bytes"] / (kern_avg_ms * 1e-3) / 1e9, 1),
            # secondary ceiling: one exponential per attended score against the exp issue rate
            "exp_ceiling": {
                "achieved": round(work["attended_scores"] / (kern_avg_ms * 1e-3) / 1e12, 3),
                "peak": round(PEAK_EXP_PER_S / 1e12, 2),
                "unit": "T exp/s",
                "frac": round(work["attended_scores"] / (kern_avg_ms * 1e-3) / PEAK_EXP_PER_S, 4),
            },
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(prob, out, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
