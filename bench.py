#!/usr/bin/env python3
"""Throughput of one GPU's sharded AdamW step (ZeRO / FSDP) on MI355X.

A step is one pass of the whole hot path over one synthetic batch: the
reduce-scatter's local reduction of the N_d ranks' bf16 gradient slices to
an fp32 mean with this shard's squared norm (clip pass), then the fused
clip + AdamW + bf16 cast/pack into the all-gather slot.  Inputs are drawn by
the seeded generator directly in HBM before timing starts.

Default workload: one GPU's ZeRO-2 shard of a 7B model over 8 ranks (875M
parameters, 8 bf16 gradient slices, global clip 1.0, t = 1000).

Prints ONE JSON line.  Only one GPU is supported: --gpus above 1 exits.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E, published
METRIC = "G params/s and achieved HBM GB/s (% of peak) for one shard's AdamW step"
KERNEL_SRC = os.path.join(ROOT, "fsdp_sharded_optimizer_zero_amd", "csrc", "zs_kernels.hip")


def kernel_source_sha() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def load_traffic(workload: str, kernel_prefix: str):
    """HBM bytes per launch of the dominant kernel (FETCH_SIZE + WRITE_SIZE,
    scaled by the plain copy's reading, averaged over its dispatches) from the
    committed counter summary of this workload, if it was taken on the current
    kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"hbm_counters_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        p = json.load(f)
    if p.get("kernel_src_sha") != kernel_source_sha():
        return None
    hits = [v for k, v in p.get("kernels", {}).items() if k.startswith(kernel_prefix + "<")]
    if not hits:
        return None
    # mean over the dispatches of every instantiation (micro-batch passes differ)
    calls = [v.get("calls", 1) for v in hits]
    return sum(v["hbm_bytes_per_dispatch"] * c for v, c in zip(hits, calls)) / sum(calls)


def host_cpu():
    """The host processor the oracle ran on: model name and logical CPUs."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "logical_cpus": os.cpu_count()}


def cpu_baseline(wl, shard, seconds: float):
    """The oracle as it stands (single thread) on a bounded sample of the same
    shard: O1..O5 over consecutive 4M-parameter chunks until `seconds` of
    oracle time; input generation is not timed."""
    import numpy as np

    import oracle as O
    import zsgen
    from zsgen.workloads import (STREAM_EXP_AVG, STREAM_EXP_AVG_SQ, STREAM_MASTER,
                                 grad_key, grad_stream)

    h = O.Hparams(lr=wl.lr, beta1=wl.beta1, beta2=wl.beta2, eps=wl.eps,
                  weight_decay=wl.weight_decay, step=wl.t0, max_grad_norm=wl.max_grad_norm)
    chunk = 1 << 22
    done, spent = 0, 0.0
    acc = O.SqAcc()
    off, V = shard.shard_offset, shard.valid_len
    m_count = wl.micro_batches
    weights = O.token_weights(wl.rank_tokens) if wl.rank_tokens else None

    def slices(j, n):
        key = grad_key(wl.t0, j, m_count)
        if wl.grad_dtype == "f32":
            return [zsgen.host_f32(wl.seed, grad_stream(0), r, key, wl.grad_sigma, off + done, n)
                    for r in range(wl.n_d)]
        return [zsgen.host_bf16(wl.seed, grad_stream(0), r, key, wl.grad_sigma, off + done, n,
                                p_out=wl.outlier_p, sigma_out=wl.outlier_sigma)
                for r in range(wl.n_d)]

    def reduce(sl):
        if weights is not None:
            return O.reduce_weighted(sl, weights)
        return O.reduce_mean_f32(sl) if wl.grad_dtype == "f32" else O.reduce_mean(sl)

    while spent < seconds and done < V:
        n = min(chunk, V - done)
        sls = [slices(j, n) for j in range(m_count)]
        w = zsgen.host_f32(wl.seed, STREAM_MASTER, 0, 0, wl.master_sigma, off + done, n)
        m = (np.zeros(n, np.float32) if wl.m_sigma is None else
             zsgen.host_f32(wl.seed, STREAM_EXP_AVG, 0, 0, wl.m_sigma, off + done, n))
        v = (np.zeros(n, np.float32) if wl.v_sigma is None else
             zsgen.host_f32(wl.seed, STREAM_EXP_AVG_SQ, 0, 0, wl.v_sigma, off + done, n,
                            absval=True))
        t0 = time.perf_counter()
        if m_count == 1:
            g = reduce(sls[0])
        else:
            g = np.empty(n, np.float32)
            for j in range(m_count):
                O.accumulate(reduce(sls[j]), j, m_count, g)
        acc.add(g)
        coef = O.clip_coef(acc.value(), wl.max_grad_norm) if wl.max_grad_norm > 0 else None
        O.adamw_f32(h, g, w, m, v, coef=coef)
        O.pack(n, w)
        spent += time.perf_counter() - t0
        done += n
    what = (f"token-weighted sum of {wl.n_d} {wl.grad_dtype} slices" if weights is not None
            else f"rank-order mean of {wl.n_d} {wl.grad_dtype} slices")
    if m_count > 1:
        what += f", accumulated over {m_count} micro-batches"
    return {"value": done / spent / 1e9, "unit": "G params/s", "cores": 1, "kind": "oracle",
            "host": host_cpu(),
            "sample": (f"oracle O1-O5 ({what}, fp64 "
                       f"exact squared norm, clip, fp32 AdamW, bf16 pack) on the first {done:,} "
                       f"of the {V:,} shard parameters of workload {wl.name}, single "
                       f"thread, {spent:.1f} s of oracle time; input generation untimed"),
            "seconds": spent}


def bench_lib():
    """The benchmark-only kernels (libzs_benchcopy.so, not part of the ABI)."""
    import ctypes as C
    lib = C.CDLL(os.path.join(ROOT, "fsdp_sharded_optimizer_zero_amd", "libzs_benchcopy.so"))
    lib.zs_bench_copy.argtypes = [C.c_void_p, C.c_void_p, C.c_int64, C.c_int32, C.c_void_p]
    lib.zs_bench_copy.restype = C.c_int
    lib.zs_bench_step_pattern.argtypes = [C.c_void_p] * 5 + [C.c_int64, C.c_int32, C.c_void_p]
    lib.zs_bench_step_pattern.restype = C.c_int
    return lib


def step_pattern_without_arithmetic(torch, run, reps=10):
    """The step's access pattern without its arithmetic (k_step_pattern), on
    the arrays of the workload's first unit: fp32 gradient, w, m, v in, w, m,
    v and the bf16 slot out, over the first multiple of 2048 parameters, in
    one-wave blocks of 4 parameters per lane at ten (the step's residency)
    and at sixteen per CU.  GB/s at 30 bytes per parameter.  It shows whether
    the step's arithmetic costs time: the step runs as fast as these accesses
    alone, or faster (its arithmetic spaces out the requests).
    Only for steps that read a stored fp32 gradient and stream (the pattern
    of the dominant kernel there); runs after the timed region and leaves the
    state changed."""
    d = run.units_data[0]
    n = run.V // 2048 * 2048
    if d.mean is None or n == 0:
        return None
    lib = bench_lib()
    out = d.out.data_ptr() + 2 * (run.shard.shard_offset if run.wl.out_mode == "gather" else 0)
    st = torch.cuda.current_stream()
    res = {}
    for per_cu in (10, 16):
        args = (d.mean.data_ptr(), d.w.data_ptr(), d.m.data_ptr(), d.v.data_ptr(), out, n,
                per_cu, st.cuda_stream)
        assert lib.zs_bench_step_pattern(*args) == 0
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(reps):
            assert lib.zs_bench_step_pattern(*args) == 0
        e1.record(st)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        res[f"per_cu_{per_cu}"] = {"ms": ms, "gbps": 30 * n / (ms / 1e3) / 1e9}
    best = max(res.values(), key=lambda r: r["gbps"])
    return {"params": n, "gbps": best["gbps"], **res}


def graph_replay(torch, run, t, steps, per_graph=20):
    """`per_graph` whole steps (t, t+1, ...) captured into one HIP graph
    (after zs_init) and the graph replayed until at least `steps` steps ran:
    the rate without host launch overhead, for steps short enough that
    launches show.  Each step's constants are frozen at capture; a replay
    repeats them on the evolving state.  A graph of one step would mostly
    time the graph launch itself, which on this runtime costs more than a
    few-microsecond kernel."""
    import fsdp_sharded_optimizer_zero_amd as Z
    Z.zs_init()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(per_graph):
            run.step(t + i)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    reps = max(1, -(-steps // per_graph))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (reps * per_graph)
    return {"ms_per_step": ms, "value": run.V * run.units / (ms / 1e3) / 1e9,
            "unit": "G params/s", "steps": reps * per_graph, "steps_per_graph": per_graph}


def copy_ceiling(torch, nbytes=4 << 30, reps=10):
    """Practical HBM bandwidth of a 16-byte-vector copy (read + write) with
    non-temporal loads and sc1 + nt stores (the streaming step's store
    policy), launched one-shot: the fastest copy measured on MI355X."""
    lib = bench_lib()
    src = torch.empty(nbytes // 2, dtype=torch.int16, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    st = torch.cuda.current_stream()
    n16 = nbytes // 16
    blocks = (n16 + 255) // 256         # one-shot: one 16-byte vector per thread
    best = None
    for _ in range(2):
        assert lib.zs_bench_copy(src.data_ptr(), dst.data_ptr(), n16, blocks, st.cuda_stream) == 0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(reps):
        assert lib.zs_bench_copy(src.data_ptr(), dst.data_ptr(), n16, blocks, st.cuda_stream) == 0
    e1.record(st)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    best = 2 * nbytes / (ms / 1e3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return {"gbps": best, "bytes_each_way": nbytes, "ms": ms}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="zero2_7b")
    ap.add_argument("--schedule", choices=["mean", "reread"], default="mean",
                    help="clip schedule: store the fp32 mean (default) or re-read the slices")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-copy-ceiling", action="store_true")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py times one GPU's shard step only (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE {world}); the exchange between GPUs is not implemented, so runs "
              "on several GPUs are not supported.", flush=True)
        sys.exit(2)

    import torch

    import fsdp_sharded_optimizer_zero_amd as Z
    from fsdp_sharded_optimizer_zero_amd.runner import ShardRun
    from zsgen.workloads import WORKLOADS

    Z.lib()                     # fail loudly if the HIP library is missing
    wl = WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    run = ShardRun(wl, store_mean=(args.schedule == "mean") if wl.max_grad_norm > 0 else None)
    run.fill_state()
    run.fill_grads(wl.t0)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    t = wl.t0
    for _ in range(args.warmup):
        run.step(t, stream=stream.cuda_stream)
        t += 1
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for k in range(K):
        ev[k][0].record(stream)
        if run.has_reduce_pass:
            run.reduce_pass(stream=stream.cuda_stream)
        ev[k][1].record(stream)
        run.update_pass(t, stream=stream.cuda_stream)
        ev[k][2].record(stream)
        t += 1
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0

    red_each = [e[0].elapsed_time(e[1]) for e in ev]
    upd_each = [e[1].elapsed_time(e[2]) for e in ev]
    red_ms = sum(red_each) / K
    upd_ms = sum(upd_each) / K
    span_ms = ev[0][0].elapsed_time(ev[-1][2]) / K
    ms_per_step = wall / K * 1e3
    params = run.V * run.units
    red_b, upd_b = run.algorithmic_bytes()
    step_gbps = (red_b + upd_b) / (ms_per_step / 1e3) / 1e9

    # dominant kernel: the fused step (k_step, one launch per unit per step)
    # or the reduction (k_reduce_sqnorm, one launch per unit and micro-batch)
    if upd_ms >= red_ms or not run.has_reduce_pass:
        kname = ("k_step (fp32 gradient in, AdamW, bf16 pack)" if run.store_mean
                 else "k_step (bf16 slices in, AdamW, bf16 pack)")
        launches = run.units
        launch_ms = upd_ms / launches
        launch_bytes = upd_b / launches
    else:
        kname = ("k_reduce_sqnorm + k_sqnorm_groups + k_sqnorm_final (rank-order reduction, "
                 "fp64 squared norm)")
        launches = run.units * run.micro
        launch_ms = red_ms / launches
        launch_bytes = red_b / launches
    achieved = launch_bytes / (launch_ms / 1e3) / 1e9
    traffic = load_traffic(wl.name, "k_step" if kname.startswith("k_step") else
                           "k_reduce_sqnorm")
    # the same figures as medians over windows of consecutive timed steps
    # (run-to-run steadiness inside this process)
    import statistics
    W = 5 if K >= 10 else max(1, K)
    wins = [(sum(red_each[i:i + W]) / W, sum(upd_each[i:i + W]) / W)
            for i in range(0, K - W + 1, W)]
    dom_idx = 1 if kname.startswith("k_step") else 0
    dom_frac = [(launch_bytes * launches) / (w[dom_idx] / 1e3) / 1e9 / PEAK_HBM_GBPS
                for w in wins]
    whole_frac = [(red_b + upd_b) / ((w[0] + w[1]) / 1e3) / 1e9 / PEAK_HBM_GBPS for w in wins]
    windows = {"steps_per_window": W, "windows": len(wins),
               "dominant_kernel_frac_median": statistics.median(dom_frac),
               "dominant_kernel_frac_min": min(dom_frac),
               "dominant_kernel_frac_max": max(dom_frac),
               "kernels_whole_step_frac_median": statistics.median(whole_frac)}

    out = {
        "metric": METRIC,
        "value": params / (ms_per_step / 1e3) / 1e9,
        "unit": "G params/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "psi": wl.psi, "n_d": wl.n_d, "rank": run.rank,
                   "stage": wl.stage, "units": run.units, "shard_params": params,
                   "max_grad_norm": wl.max_grad_norm, "grad_dtype": wl.grad_dtype,
                   "rank_tokens": list(wl.rank_tokens) or None,
                   "micro_batches": wl.micro_batches,
                   "schedule": ("stored-mean" if run.store_mean else "reread")
                   if run.has_reduce_pass else "fused"},
        "hbm_gbps": step_gbps,
        "hbm_frac_of_peak": step_gbps / PEAK_HBM_GBPS,
        "algorithmic_bytes_per_step": red_b + upd_b,
        "kernel_ms": {"clip_pass": red_ms, "update_pass": upd_ms, "event_span_per_step": span_ms},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBPS, "traffic": traffic, "kernel": kname,
                     "algorithmic_bytes_per_launch": launch_bytes, "launch_ms": launch_ms,
                     "launches_per_step": launches},
        "windows": windows,
        "kernel_src_sha": kernel_source_sha(),
    }
    if ms_per_step < 1.0:
        out["graph_replay"] = graph_replay(torch, run, t, K)
    if not args.no_copy_ceiling:
        pattern = step_pattern_without_arithmetic(torch, run) if (run.store_mean and kname.startswith(
            "k_step") and launch_bytes >= (512 << 20)) else None
        del run
        torch.cuda.empty_cache()
        cc = copy_ceiling(torch)
        out["copy_ceiling"] = cc
        ratios = {"dominant_kernel_over_copy": achieved / cc["gbps"],
                  "kernels_whole_step_over_copy": (red_b + upd_b) / ((red_ms + upd_ms) / 1e3)
                  / 1e9 / cc["gbps"]}
        if pattern is not None:
            out["step_pattern_without_arithmetic"] = pattern
            ratios["k_step_over_step_pattern"] = achieved / pattern["gbps"]
            ratios["step_pattern_over_copy"] = pattern["gbps"] / cc["gbps"]
        out["ceiling_ratios"] = ratios
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, Z.zs_layout(
            wl.psi, wl.n_d, wl.rank, wl.align, wl.stage,
            Z.ZS_OUT_GATHER if wl.out_mode == "gather" else Z.ZS_OUT_SHARD), args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
