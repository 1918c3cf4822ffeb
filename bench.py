#!/usr/bin/env python3
"""Benchmark of the causal dynamic short convolution on one MI355X.

A step is one forward plus one backward pass over one batch of the workload,
through the library's C-ABI entry points (dsc_fwd + dsc_bwd, or the low-rank
pair). Inputs are drawn (seeded, synthetic) and copied to HBM before timing.
W untimed warm-up steps, then exactly K timed steps between two
synchronisations. Prints one JSON line.

  value      tokens/s of the timed steps (B*T per step)
  roofline   the dominant launch's algorithmic bytes (or, where the matrix
             cores bound it, algorithmic MFMA flops) over its average launch
             time (HIP events on the launch stream around every launch of the
             timed steps), against the 8 TB/s HBM3E
             peak (or 2.5 PFLOP/s dense bf16); `traffic` from the committed
             rocprofv3 counter summary when it matches the current kernel source
  cpu_baseline  the CPU oracle on the host cores, on the same workload
  configs    (default workload only) every one of the five configurations the
             method is specified on, timed on the GPU alone in the same way
             (--config-steps, --config-warmup), each with its own roofline
  hosts      (default workload only) the same for the short convolutions of the
             Mamba-2 and Gated DeltaNet hosts (one filter per channel)
  other_paths  (default workload only) the same for the R=32 low-rank layer in
             fp32 (vector-ALU kernels: roofline against the fp64 vector peak,
             their long sums running in double) and the QKV layer with
             24-channel filter heads

Decode workloads (--workload decode_*) time the decode step instead: one new
token for each of B rows through one layer (dsc_decode_step or
dsc_lowrank_decode_step). A step is one replay of a HIP graph holding that call
for L layers, each with its own inputs, ring and (low-rank) U, L chosen so the
layers' buffers exceed 1 GiB and every step reads them from HBM rather than
the 256 MB last-level cache. value is rows/s through one layer (B*L per step).

The generator workload (--workload gen_qkv_headwise_bf16) times the forward with
filters generated in the kernel (dsc_fwd_gen) from a hidden state of width K; a
step is one such launch. It also times the unfused pair (torch's GEMM writing
bf16 filters, then dsc_fwd) for comparison; its roofline is the matrix cores.
Beside it (key "backward") the fused backward dsc_bwd_gen and the unfused
GEMM + dsc_bwd pair are timed the same way.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
FP64_VECTOR_PEAK_TFLOPS = 78.6
DEFAULT_WORKLOAD = "qkv_headwise_bf16"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def algorithmic_bytes(wl) -> dict:
    """Bytes the method must move per token (each tensor read or written once)."""
    e = 2 if wl.dtype == "bf16" else 4
    if wl.kind == "headwise":
        fwd = 2 * wl.D * e + wl.G * wl.W * e                 # x, w in; y out
        bwd = 3 * wl.D * e + 2 * wl.G * wl.W * e             # x, w, dy in; dx, dw out
        fixed_fwd = fixed_bwd = 0
    else:
        fwd = 2 * wl.D * e + wl.R * e                        # x, z in; y out
        bwd = 3 * wl.D * e + 2 * wl.R * e                    # x, z, dy in; dx, dz out
        fixed_fwd = wl.R * wl.D * wl.W * e                   # U in
        fixed_bwd = 2 * wl.R * wl.D * wl.W * e               # U in, dU out
    if wl.packed_mean > 0:  # the positions, read once by each pass
        fwd += 4
        bwd += 4
    n = wl.tokens
    return {"fwd": fwd * n + fixed_fwd, "bwd": bwd * n + fixed_bwd,
            "fwd_per_token": fwd, "bwd_per_token": bwd}


def algorithmic_mfma_flops(wl) -> dict:
    """Dense contractions of the low-rank form, 2*B*T*R*D*W flops each: the filter
    generation z.U (forward; regenerated in the backward, since the filters are never
    stored), and dz and dU in the backward (on the matrix cores in bf16, on the vector
    ALUs in fp32). The convolution itself and the head-wise form are vector work and
    are not counted."""
    if wl.kind != "lowrank":
        return {"fwd": 0, "bwd": 0}
    one = 2 * wl.tokens * wl.R * wl.D * wl.W
    return {"fwd": one, "bwd": 3 * one}


# The sources each kernel family is built from: a recorded traffic figure is only
# reported while these files are unchanged.
KERNEL_SOURCES = {
    "headwise": ["common.hpp", "headwise_kernels.hpp", "headwise_dispatch.hpp", "headwise_bf16.hip"],
    "lowrank": ["common.hpp", "lowrank_mfma.hpp", "lowrank_bwd_tr.hpp", "lowrank_mfma_dispatch.hpp",
                "lowrank_plan.hpp", "lowrank.hip", "buffer.hpp"]
               + [f"lowrank_{d}_w{w}.hip" for d in ("fwd", "bwd", "bwd_pos") for w in range(1, 9)],
    "decode": ["common.hpp", "buffer.hpp", "lowrank_mfma.hpp", "decode.hip"],
    "gen": ["common.hpp", "buffer.hpp", "lowrank_mfma.hpp", "headwise_kernels.hpp", "gen.hip"],
}


def kernel_source_digest(kind: str) -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "dynamic_short_convolutions_amd", "csrc")
    for name in KERNEL_SOURCES[kind]:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def measured_traffic(kind: str, kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary, or None if absent or stale."""
    try:
        with open(TRAFFIC_FILE) as f:
            tab = json.load(f)
    except (OSError, ValueError):
        return None
    rec = tab.get(f"{workload}:{kernel}")
    if not rec or rec.get("source_digest") != kernel_source_digest(kind):
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(wl, inp, min_seconds: float, max_reps: int) -> dict:
    import numpy as np

    import oracle

    oracle.build(force=False)
    threads = oracle.get_threads()
    one = one_core_rate(wl, inp)
    if wl.kind == "headwise":
        # whole batch, repeated until min_seconds have passed
        reps, t0 = 0, time.perf_counter()
        if wl.rope_head_dim > 0:
            from dynamic_short_convolutions_amd.synthetic import rope_table

            cos, sin = rope_table(wl.T, wl.rope_head_dim)
            rope_args = (cos, sin, wl.rope_d_rot, wl.rope_head_dim, wl.rope_interleaved)
        while True:
            if wl.rope_head_dim > 0:
                oracle.fwd_rope(inp["x"], inp["w"], wl.residual, *rope_args, pos=inp.get("pos"))
                oracle.bwd_rope(inp["x"], inp["w"], inp["dy"], wl.residual, *rope_args, pos=inp.get("pos"))
            else:
                oracle.fwd(inp["x"], inp["w"], wl.residual, pos=inp.get("pos"))
                oracle.bwd(inp["x"], inp["w"], inp["dy"], wl.residual, pos=inp.get("pos"))
            reps += 1
            el = time.perf_counter() - t0
            if el >= min_seconds or reps >= max_reps:
                break
        return {"value": reps * wl.tokens / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
                "sample": f"{reps} full forward+backward pass(es) over the whole {wl.B}x{wl.T} batch, "
                          f"{el:.1f} s, OpenMP over output rows", **one}
    # low-rank: a full pass takes minutes to hours, so time the per-token outputs (y, dx, dz)
    # on a sample of tokens and dU on a sample of columns, and scale each to the whole batch
    rng = np.random.default_rng(1)
    n_rows = max(16, int(wl.tokens * 2048 / (wl.D * wl.W * wl.R)) // 8 * 8)
    rows = rng.choice(wl.tokens, size=min(n_rows, wl.tokens), replace=False)
    t0 = time.perf_counter()
    oracle.lowrank_fwd(inp["x"], inp["z"], inp["U"], wl.W, wl.residual, rows=rows, pos=inp.get("pos"))
    oracle.lowrank_bwd_rows(inp["x"], inp["z"], inp["U"], inp["dy"], wl.W, wl.residual, rows=rows, pos=inp.get("pos"))
    t_rows = time.perf_counter() - t0
    ncols = wl.D * wl.W
    cols = rng.choice(ncols, size=min(64, ncols), replace=False)
    t0 = time.perf_counter()
    oracle.lowrank_dU(inp["x"], inp["z"], inp["dy"], wl.W, cols=cols, pos=inp.get("pos"))
    t_cols = time.perf_counter() - t0
    est = t_rows * wl.tokens / rows.size + t_cols * ncols / cols.size
    return {"value": wl.tokens / est, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"y, dx and dz on {rows.size} random tokens ({t_rows:.1f} s) and dU on {cols.size} "
                      f"random columns over all tokens ({t_cols:.1f} s), scaled to the whole "
                      f"{wl.B}x{wl.T} batch (estimated {est:.0f} s for one pass)", **one}


def one_core_rate(wl, inp) -> dict:
    """The oracle on one thread, on a small sample of tokens (and of dU columns), scaled
    to tokens/s like the all-cores figure."""
    import numpy as np

    import oracle

    threads = oracle.get_threads()
    rng = np.random.default_rng(2)
    oracle.set_threads(1)
    try:
        if wl.rope_head_dim > 0:
            # the rotary oracle rotates whole tensors: time it on the first 256 tokens of one sequence
            from dynamic_short_convolutions_amd.synthetic import rope_table

            n = min(256, wl.T)
            sub = {k: np.ascontiguousarray(inp[k][:1, :n]) for k in ("x", "w", "dy")}
            cos, sin = rope_table(wl.T, wl.rope_head_dim)
            args = (cos, sin, wl.rope_d_rot, wl.rope_head_dim, wl.rope_interleaved)
            t0 = time.perf_counter()
            oracle.fwd_rope(sub["x"], sub["w"], wl.residual, *args)
            oracle.bwd_rope(sub["x"], sub["w"], sub["dy"], wl.residual, *args)
            el = time.perf_counter() - t0
            rate, what = n / el, f"the first {n} tokens of one sequence, forward+backward with rotation, {el:.1f} s"
        elif wl.kind == "headwise":
            rows = rng.choice(wl.tokens, size=min(512, wl.tokens), replace=False)
            t0 = time.perf_counter()
            oracle.fwd(inp["x"], inp["w"], wl.residual, rows=rows, pos=inp.get("pos"))
            oracle.bwd(inp["x"], inp["w"], inp["dy"], wl.residual, rows=rows, pos=inp.get("pos"))
            el = time.perf_counter() - t0
            rate, what = rows.size / el, f"{rows.size} random tokens, forward+backward, {el:.1f} s"
        else:
            n_rows = max(8, int(wl.tokens * 256 / (wl.D * wl.W * wl.R)) // 8 * 8)
            rows = rng.choice(wl.tokens, size=min(n_rows, wl.tokens), replace=False)
            t0 = time.perf_counter()
            oracle.lowrank_fwd(inp["x"], inp["z"], inp["U"], wl.W, wl.residual, rows=rows, pos=inp.get("pos"))
            oracle.lowrank_bwd_rows(inp["x"], inp["z"], inp["U"], inp["dy"], wl.W, wl.residual, rows=rows,
                                    pos=inp.get("pos"))
            t_rows = time.perf_counter() - t0
            ncols = wl.D * wl.W
            cols = rng.choice(ncols, size=min(4, ncols), replace=False)
            t0 = time.perf_counter()
            oracle.lowrank_dU(inp["x"], inp["z"], inp["dy"], wl.W, cols=cols, pos=inp.get("pos"))
            t_cols = time.perf_counter() - t0
            est = t_rows * wl.tokens / rows.size + t_cols * ncols / cols.size
            rate, what = wl.tokens / est, (f"{rows.size} random tokens ({t_rows:.1f} s) and dU on {cols.size} "
                                           f"columns ({t_cols:.1f} s), scaled to the batch")
    finally:
        oracle.set_threads(threads)
    return {"value_1core": rate, "sample_1core": what}


def decode_bytes(wl) -> dict:
    """Bytes one decode call must move with every row active and its ring full: x, the
    W-1 ring slots, the filter (w, or z and once per call U) and pos read; y and one
    ring slot written."""
    e = 2 if wl.dtype == "bf16" else 4
    filt = wl.G * wl.W * e if wl.kind == "headwise" else wl.R * e
    per_row = (wl.D + (wl.W - 1) * wl.D + wl.D + wl.D) * e + filt + 4
    fixed = wl.R * wl.D * wl.W * e if wl.kind == "lowrank" else 0
    return {"per_row": per_row, "fixed": fixed, "per_call": per_row * wl.B + fixed}


def decode_cpu_baseline(wl, inp, min_seconds: float, max_reps: int) -> dict:
    import oracle

    oracle.build(force=False)
    threads = oracle.get_threads()
    reps, t0 = 0, time.perf_counter()
    while True:
        if wl.kind == "headwise":
            oracle.decode_step(inp["x"], inp["w"], inp["pos"], inp["state"], wl.residual)
        else:
            oracle.lowrank_decode_step(inp["x"], inp["z"], inp["U"], inp["pos"], inp["state"], wl.W, wl.residual)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds or reps >= max_reps:
            break
    return {"value": reps * wl.B / el, "unit": "rows/s", "cores": threads, "kind": "oracle",
            "sample": f"{reps} decode step(s) over all {wl.B} rows, {el:.1f} s, OpenMP over rows"}


def decode_main(a, wl) -> int:
    import math

    import numpy as np
    import torch

    import dynamic_short_convolutions_amd as dsc
    from dynamic_short_convolutions_amd.synthetic import draw_decode

    print(f"[bench] drawing {wl.name}", file=sys.stderr, flush=True)
    inp = draw_decode(wl)
    nb = decode_bytes(wl)

    def dev(arr):
        if arr.dtype == np.uint16:
            return torch.from_numpy(arr.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(arr).cuda()

    base = {k: dev(v) for k, v in inp.items()}
    base["y"] = torch.empty_like(base["x"])
    set_bytes = sum(v.numel() * v.element_size() for v in base.values())
    layers = max(1, math.ceil((1 << 30) / set_bytes))
    sets = []
    for _ in range(layers):
        sets.append({k: v.clone() for k, v in base.items()})

    def call(b):
        if wl.kind == "headwise":
            dsc.dsc_decode_step(b["x"], b["w"], b["pos"], b["state"], b["y"], wl.residual)
        else:
            dsc.dsc_lowrank_decode_step(b["x"], b["z"], b["U"], b["pos"], b["state"], b["y"], wl.W, wl.residual)

    def run_all():
        for b in sets:
            call(b)

    print(f"[bench] {layers} layers of buffers, capturing the decode graph", file=sys.stderr, flush=True)
    run_all()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run_all()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run_all()
    for _ in range(a.warmup):
        g.replay()
    torch.cuda.synchronize()
    print(f"[bench] timing {a.steps} steps", file=sys.stderr, flush=True)
    # HIP events on the replay stream around every replay of the timed region: a
    # replay runs the layers' decode kernels back to back, so a replay's duration over
    # the layer count is the kernel's average duration (a kernel trace agrees)
    stream = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(a.steps + 1)]
    t0 = time.perf_counter()
    evs[0].record(stream)
    for i in range(a.steps):
        g.replay()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    ms_step = el / a.steps * 1e3
    ms_call = ms_step / layers
    per = sorted(evs[i].elapsed_time(evs[i + 1]) / layers for i in range(a.steps))
    launch_ms = evs[0].elapsed_time(evs[-1]) / (a.steps * layers)
    pct = {"p10": per[int(0.1 * (len(per) - 1))], "p50": per[(len(per) - 1) // 2],
           "p90": per[int(0.9 * (len(per) - 1))]}
    kern = "headwise_decode_kernel" if wl.kind == "headwise" else "lowrank_decode_mfma_kernel"
    achieved = nb["per_call"] / (launch_ms * 1e-3) / 1e9

    cpu = None
    if not a.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        cpu = decode_cpu_baseline(wl, inp, a.cpu_seconds, 100000)

    out = {
        "metric": "dyn-shortconv decode step: rows/s through one layer and HBM GB/s (% of peak)",
        "value": wl.B / (ms_call * 1e-3),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded i.i.d. Gaussian; positions uniform in [W-1, 4096))",
        "config": {"workload": wl.name, "B": wl.B, "D": wl.D, "W": wl.W,
                   **({"Hc": wl.Hc} if wl.kind == "headwise" else {"R": wl.R}),
                   "residual": wl.residual, "layers_per_step": layers, "accumulate": "f32",
                   "parallelism": "single GPU", "timing": "HIP graph replay of one step"},
        "us_per_call": ms_call * 1e3,
        "hbm_GBps": nb["per_call"] / (ms_call * 1e-3) / 1e9,
        "hbm_frac_of_peak": nb["per_call"] / (ms_call * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "launch_ms": launch_ms,
        "launch_ms_percentiles": pct,
        "algorithmic_bytes": nb,
        "roofline": {"bound": "hbm", "kernel": kern, "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": measured_traffic("decode", kern, wl.name)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))
    return 0


def gen_main(a, wl) -> int:
    """The forward with filters generated in the kernel (dsc_fwd_gen), against the
    unfused path: torch's GEMM (hipBLASLt) writing bf16 filters, then dsc_fwd."""
    import numpy as np
    import torch

    import dynamic_short_convolutions_amd as dsc
    from dynamic_short_convolutions_amd.synthetic import draw_gen

    K = wl.gen_hidden
    print(f"[bench] drawing {wl.name}", file=sys.stderr, flush=True)
    inp = draw_gen(wl, K)
    dev = lambda arr: torch.from_numpy(arr.view(np.int16)).cuda().view(torch.bfloat16)
    x, h, Wg = dev(inp["x"]), dev(inp["h"]), dev(inp["Wg"])
    y = torch.empty_like(x)
    WgT = Wg.t().contiguous()
    w = torch.empty((wl.B, wl.T, wl.G, wl.W), dtype=torch.bfloat16, device="cuda")
    fused = lambda: dsc.dsc_fwd_gen(x, h, Wg, y, wl.W, wl.residual)
    gemm = lambda: torch.matmul(h.reshape(-1, K), WgT, out=w.view(-1, wl.G * wl.W))
    conv = lambda: dsc.dsc_fwd(x, w, y, wl.residual)
    stream = torch.cuda.current_stream()

    def timed(fn, reps):
        """reps back-to-back launches with a HIP event between consecutive ones"""
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        evs[0].record(stream)
        for e_ in evs[1:]:
            fn()
            e_.record(stream)
        torch.cuda.synchronize()
        t = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(reps))
        return sum(t) / len(t), {"p10": t[int(0.1 * (len(t) - 1))], "p50": t[(len(t) - 1) // 2],
                                 "p90": t[int(0.9 * (len(t) - 1))]}

    for _ in range(a.warmup):
        fused()
        gemm()
        conv()
    torch.cuda.synchronize()
    print(f"[bench] timing {a.steps} steps", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    launch_ms, pct = timed(fused, a.steps)  # events around every launch of the timed steps
    ms_step = (time.perf_counter() - t0) / a.steps * 1e3
    # the unfused pair as a caller would run it: the GEMM, then the convolution reading
    # its filters, back to back, with an event between consecutive launches
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * a.launch_reps + 1)]
    evs[0].record(stream)
    for i in range(a.launch_reps):
        gemm()
        evs[2 * i + 1].record(stream)
        conv()
        evs[2 * i + 2].record(stream)
    torch.cuda.synchronize()
    gemm_ms = sum(evs[2 * i].elapsed_time(evs[2 * i + 1]) for i in range(a.launch_reps)) / a.launch_reps
    conv_ms = sum(evs[2 * i + 1].elapsed_time(evs[2 * i + 2]) for i in range(a.launch_reps)) / a.launch_reps
    flops = 2.0 * wl.tokens * K * wl.G * wl.W
    hbm = wl.tokens * (2 * wl.D + K) * 2 + wl.G * wl.W * K * 2  # x, h in; y out; Wg once
    achieved = flops / (launch_ms * 1e-3) / 1e12
    # the backward through the convolution: dx and the filters' gradient dw, fused (filters
    # regenerated in the kernel) against the GEMM + dsc_bwd pair (dh = dw.Wg and
    # dWg = dw^T.h follow in both cases and are not timed)
    g = torch.Generator(device="cuda")
    g.manual_seed(20261215)
    dy = torch.randn(x.shape, device="cuda", generator=g, dtype=torch.float32).to(torch.bfloat16)
    dx, dw = torch.empty_like(x), torch.empty_like(w)
    fused_bwd = lambda: dsc.dsc_bwd_gen(x, h, Wg, dy, dx, dw, wl.W, wl.residual)
    conv_bwd = lambda: dsc.dsc_bwd(x, w, dy, dx, dw, wl.residual)
    for _ in range(a.warmup):
        fused_bwd()
        gemm()
        conv_bwd()
    torch.cuda.synchronize()
    bwd_ms, bwd_pct = timed(fused_bwd, a.launch_reps)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * a.launch_reps + 1)]
    evs[0].record(stream)
    for i in range(a.launch_reps):
        gemm()
        evs[2 * i + 1].record(stream)
        conv_bwd()
        evs[2 * i + 2].record(stream)
    torch.cuda.synchronize()
    bgemm_ms = sum(evs[2 * i].elapsed_time(evs[2 * i + 1]) for i in range(a.launch_reps)) / a.launch_reps
    bconv_ms = sum(evs[2 * i + 1].elapsed_time(evs[2 * i + 2]) for i in range(a.launch_reps)) / a.launch_reps
    bwd_hbm = wl.tokens * (3 * wl.D + K + wl.G * wl.W) * 2 + wl.G * wl.W * K * 2  # x, dy, h in; dx, dw out
    backward = {"kernel": "gen_bwd_kernel", "launch_ms": bwd_ms, "launch_ms_percentiles": bwd_pct,
                "unfused_ms": {"gemm": bgemm_ms, "conv": bconv_ms, "total": bgemm_ms + bconv_ms},
                "algorithmic_mfma_flops": flops, "algorithmic_bytes": bwd_hbm,
                "mfma_TFLOPs": flops / (bwd_ms * 1e-3) / 1e12, "hbm_GBps": bwd_hbm / (bwd_ms * 1e-3) / 1e9,
                "traffic": measured_traffic("gen", "gen_bwd_kernel", wl.name)}
    cpu = None
    if not a.no_cpu_baseline:
        import oracle

        oracle.build(force=False)
        # a probe of 256 tokens sizes a sample of about --cpu-seconds of oracle work
        rng = np.random.default_rng(3)
        t1 = time.perf_counter()
        oracle.fwd_gen(inp["x"], inp["h"], inp["Wg"], wl.G, wl.W, wl.residual,
                       rows=rng.choice(wl.tokens, size=256, replace=False))
        n = int(min(wl.tokens, max(256, 256 * a.cpu_seconds / max(time.perf_counter() - t1, 1e-6))))
        rows = rng.choice(wl.tokens, size=n, replace=False)
        t1 = time.perf_counter()
        oracle.fwd_gen(inp["x"], inp["h"], inp["Wg"], wl.G, wl.W, wl.residual, rows=rows)
        el = time.perf_counter() - t1
        cpu = {"value": rows.size / el, "unit": "tokens/s", "cores": oracle.get_threads(), "kind": "oracle",
               "sample": f"{rows.size} random tokens (filters generated for those steps), {el:.1f} s"}
    out = {
        "metric": "dyn-shortconv forward with filters generated in the kernel: tokens/s",
        "value": wl.tokens / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic (seeded i.i.d. Gaussian)",
        "config": {"workload": wl.name, "B": wl.B, "T": wl.T, "D": wl.D, "W": wl.W, "Hc": wl.Hc, "K": K,
                   "residual": wl.residual, "accumulate": "f32", "parallelism": "single GPU", "pass": "forward"},
        "launch_ms": launch_ms, "launch_ms_percentiles": pct,
        "unfused_ms": {"gemm": gemm_ms, "conv": conv_ms, "total": gemm_ms + conv_ms},
        "algorithmic_mfma_flops": flops, "algorithmic_bytes": hbm,
        "hbm_GBps": hbm / (launch_ms * 1e-3) / 1e9,
        "roofline": {"bound": "mfma", "kernel": "gen_fwd_kernel", "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / MFMA_BF16_PEAK_TFLOPS,
                     "traffic": measured_traffic("gen", "gen_fwd_kernel", wl.name)},
        "cpu_baseline": cpu,
        "backward": backward,
    }
    print(json.dumps(out))
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--launch-reps", type=int, default=20,
                    help="event-timed repetitions of the generator workload's backward and of the unfused "
                         "GEMM + forward / backward pairs it is compared with")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="seconds of CPU oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="default workload only: skip the GPU-only timing of the other four configurations "
                         "and of the linear-RNN host shapes")
    ap.add_argument("--config-steps", type=int, default=10, help="timed steps per extra configuration")
    ap.add_argument("--config-warmup", type=int, default=3, help="warm-up steps per extra configuration")
    ap.add_argument("--rows", type=int, default=0, help="decode workloads: rows per call (default: the workload's)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy, fill and sum (for scaling the HBM byte counters)")
    a = ap.parse_args()

    if a.gpus != 1:
        print(f"bench.py: this library runs on one GPU; --gpus {a.gpus} is not supported "
              "(the multi-GPU sharding is a design note only)", file=sys.stderr)
        return 2

    import torch

    import dynamic_short_convolutions_amd as dsc
    from dynamic_short_convolutions_amd.synthetic import DECODE_WORKLOADS, WORKLOADS, draw

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    dsc.lib()  # fail loudly if the HIP library is missing

    if a.copy_calibration:
        # three kernels of known traffic per launch: a copy (1 GiB read + 1 GiB written),
        # a fill (1 GiB written) and a sum (1 GiB read), 5 launches each
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        for _ in range(5):
            src.fill_(3)
        total = 0
        for _ in range(5):
            total += int(src.view(torch.int64).sum())
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "fill_bytes": n, "sum_bytes": n, "launches": 5, "sum": total}))
        return 0

    if a.workload in DECODE_WORKLOADS:
        wl = DECODE_WORKLOADS[a.workload]
        return decode_main(a, dataclasses.replace(wl, B=a.rows) if a.rows > 0 else wl)
    wl = WORKLOADS[a.workload]
    if wl.gen_hidden > 0:
        return gen_main(a, wl)
    print(f"[bench] drawing {wl.name}", file=sys.stderr, flush=True)
    inp = draw(wl, need_dy=True)
    fwd, bwd, kern, keep = training_calls(wl, inp)
    m = time_training(fwd, bwd, a.steps, a.warmup)
    rec = training_record(wl, m, kern)

    cpu = None
    if not a.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl, inp, a.cpu_seconds, 1000)
    del fwd, bwd, keep, inp

    configs = hosts = others = None
    if a.workload == DEFAULT_WORKLOAD and not a.no_configs:
        configs = all_configs(a, {wl.name: (rec, m)})
        hosts = all_configs(a, {}, HOST_WORKLOADS)
        others = all_configs(a, {}, OTHER_WORKLOADS)

    out = {
        "metric": "dyn-shortconv fwd+bwd tokens/s and HBM GB/s (% of peak), D=2048 W=4 bf16",
        "value": rec["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": m["ms_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded i.i.d. Gaussian)",
        "config": {"workload": wl.name, "B": wl.B, "T": wl.T, "D": wl.D, "W": wl.W,
                   **({"Hc": wl.Hc} if wl.kind == "headwise" else {"R": wl.R}),
                   **({"packed_mean_len": wl.packed_mean} if wl.packed_mean > 0 else {}),
                   **({"rope_head_dim": wl.rope_head_dim, "rope_d_rot": wl.rope_d_rot,
                       "rope_interleaved": wl.rope_interleaved} if wl.rope_head_dim > 0 else {}),
                   "residual": wl.residual, "accumulate": "f32", "global_batch": wl.B, "seq_len": wl.T,
                   "parallelism": "single GPU"},
        "hbm_GBps": rec["hbm_GBps"],
        "hbm_frac_of_peak": rec["hbm_frac_of_peak"],
        "launch_ms": m["launch_ms"],
        "launch_ms_percentiles": m["launch_pct"],
        "algorithmic_bytes": rec["algorithmic_bytes"],
        **({"algorithmic_mfma_flops": rec["algorithmic_mfma_flops"]} if wl.kind == "lowrank" else {}),
        "roofline": rec["roofline"],
        "cpu_baseline": cpu,
        **({"configs": configs} if configs is not None else {}),
        **({"hosts": hosts} if hosts is not None else {}),
        **({"other_paths": others} if others is not None else {}),
    }
    print(json.dumps(out))
    return 0


def training_calls(wl, inp):
    """Device copies of the inputs and the forward / backward calls of a training
    workload (backward None for a forward-only one). Returns (fwd, bwd, kernel names,
    tensors to keep alive)."""
    import numpy as np
    import torch

    import dynamic_short_convolutions_amd as dsc

    def dev(arr):
        if arr.dtype == np.uint16:
            return torch.from_numpy(arr.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(arr).cuda()

    t = {k: dev(v) for k, v in inp.items() if k != "dy" or wl.backward}
    x = t["x"]
    pos = t.get("pos")  # packed sequences: positions within each sequence
    bwd = None
    if wl.kind == "headwise" and wl.rope_head_dim > 0:
        # rotary embedding of the Q and K channels fused after the convolution
        from dynamic_short_convolutions_amd.synthetic import rope_table

        w, dy = t["w"], t["dy"]
        t["y"], t["dx"], t["dw"] = torch.empty_like(x), torch.empty_like(x), torch.empty_like(w)
        cos, sin = (torch.from_numpy(a).cuda() for a in rope_table(wl.T, wl.rope_head_dim))
        t["cos"], t["sin"] = cos, sin
        rope = dsc.rope_args(cos, sin, wl.rope_d_rot, wl.rope_head_dim, wl.rope_interleaved)
        fwd = lambda: dsc.dsc_fwd_rope(x, w, pos, rope, t["y"], wl.residual)
        bwd = lambda: dsc.dsc_bwd_rope(x, w, pos, rope, dy, t["dx"], t["dw"], wl.residual)
        kern = {"fwd": "headwise_fwd_kernel", "bwd": "headwise_bwd_kernel"}
    elif wl.kind == "headwise":
        w = t["w"]
        t["y"] = torch.empty_like(x)
        if pos is None:
            fwd = lambda: dsc.dsc_fwd(x, w, t["y"], wl.residual)
        else:
            fwd = lambda: dsc.dsc_fwd_varlen(x, w, pos, t["y"], wl.residual)
        if wl.backward:
            dy = t["dy"]
            t["dx"], t["dw"] = torch.empty_like(x), torch.empty_like(w)
            if pos is None:
                bwd = lambda: dsc.dsc_bwd(x, w, dy, t["dx"], t["dw"], wl.residual)
            else:
                bwd = lambda: dsc.dsc_bwd_varlen(x, w, pos, dy, t["dx"], t["dw"], wl.residual)
        kern = {"fwd": "headwise_fwd_kernel", "bwd": "headwise_bwd_kernel"}
    else:
        z, U, dy = t["z"], t["U"], t["dy"]
        t["y"], t["dx"], t["dz"], t["dU"] = torch.empty_like(x), torch.empty_like(x), torch.empty_like(z), \
            torch.empty_like(U)
        nws = dsc.dsc_lowrank_bwd_workspace_bytes(wl.B, wl.T, wl.D, wl.R, wl.W,
                                                  dsc.DSC_BF16 if wl.dtype == "bf16" else dsc.DSC_F32)
        ws = torch.empty(max(nws, 16), dtype=torch.uint8, device="cuda") if nws else None
        t["ws"] = ws
        if pos is None:
            fwd = lambda: dsc.dsc_lowrank_fwd(x, z, U, t["y"], wl.W, wl.residual)
            bwd = lambda: dsc.dsc_lowrank_bwd(x, z, U, dy, t["dx"], t["dz"], t["dU"], ws, wl.W, wl.residual)
        else:
            fwd = lambda: dsc.dsc_lowrank_fwd_varlen(x, z, U, pos, t["y"], wl.W, wl.residual)
            bwd = lambda: dsc.dsc_lowrank_bwd_varlen(x, z, U, pos, dy, t["dx"], t["dz"], t["dU"], ws, wl.W,
                                                     wl.residual)
        kern = {"fwd": "lowrank_fwd", "bwd": "lowrank_bwd"}
    return fwd, bwd, kern, t


def time_training(fwd, bwd, steps: int, warmup: int) -> dict:
    """`warmup` untimed steps, then `steps` timed ones between two synchronisations.
    Per-launch durations come from HIP events recorded on the launch stream between
    the launches of the timed steps (event 2i before forward i, 2i+1 between it and
    backward i, 2i+2 after backward i)."""
    import torch

    passes = ("fwd", "bwd") if bwd is not None else ("fwd",)
    calls = {"fwd": fwd, "bwd": bwd}
    stream = torch.cuda.current_stream()
    print(f"[bench] warmup {warmup}", file=sys.stderr, flush=True)
    for _ in range(warmup):
        for p in passes:
            calls[p]()
    torch.cuda.synchronize()
    print(f"[bench] timing {steps} steps", file=sys.stderr, flush=True)
    n = len(passes)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n * steps + 1)]
    t0 = time.perf_counter()
    evs[0].record(stream)
    for i in range(steps):
        for j, p in enumerate(passes):
            calls[p]()
            evs[n * i + j + 1].record(stream)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    launch_ms, launch_pct = {}, {}
    for j, name in enumerate(passes):
        times = sorted(evs[n * i + j].elapsed_time(evs[n * i + j + 1]) for i in range(steps))
        launch_ms[name] = sum(times) / len(times)
        launch_pct[name] = {"p10": times[int(0.1 * (len(times) - 1))], "p50": times[(len(times) - 1) // 2],
                            "p90": times[int(0.9 * (len(times) - 1))]}
    return {"ms_step": el / steps * 1e3, "launch_ms": launch_ms, "launch_pct": launch_pct}


def training_record(wl, m: dict, kern: dict) -> dict:
    """Throughput, algorithmic HBM rate and the dominant launch against its roofline."""
    nbytes = algorithmic_bytes(wl)
    nflops = algorithmic_mfma_flops(wl)
    passes = list(m["launch_ms"])
    dom = max(passes, key=lambda k: m["launch_ms"][k])
    # the bound of the dominant launch: the larger of its HBM and matrix-core times at peak;
    # fp32 low-rank runs on the vector ALUs with its dz and dU sums (two thirds of the
    # backward's flops) in double, so its contractions are priced at the fp64 vector peak
    alu = wl.kind == "lowrank" and wl.dtype == "f32"
    mfma_bound = not alu and nflops[dom] / (MFMA_BF16_PEAK_TFLOPS * 1e12) > nbytes[dom] / (HBM_PEAK_GBPS * 1e9)
    if alu:
        achieved, peak, unit = nflops[dom] / (m["launch_ms"][dom] * 1e-3) / 1e12, FP64_VECTOR_PEAK_TFLOPS, "TFLOP/s"
    elif mfma_bound:
        achieved, peak, unit = nflops[dom] / (m["launch_ms"][dom] * 1e-3) / 1e12, MFMA_BF16_PEAK_TFLOPS, "TFLOP/s"
    else:
        achieved, peak, unit = nbytes[dom] / (m["launch_ms"][dom] * 1e-3) / 1e9, HBM_PEAK_GBPS, "GB/s"
    step_bytes = sum(nbytes[p] for p in passes)
    step_gbps = step_bytes / (m["ms_step"] * 1e-3) / 1e9
    return {
        "tokens_per_s": wl.tokens / (m["ms_step"] * 1e-3),
        "hbm_GBps": step_gbps,
        "hbm_frac_of_peak": step_gbps / HBM_PEAK_GBPS,
        "algorithmic_bytes": {p: nbytes[p] for p in passes},
        "algorithmic_mfma_flops": {p: nflops[p] for p in passes},
        "roofline": {"bound": "alu" if alu else ("mfma" if mfma_bound else "hbm"), "kernel": kern[dom],
                     "achieved": achieved,
                     "peak": peak, "unit": unit, "frac": achieved / peak,
                     "traffic": measured_traffic(wl.kind, kern[dom], wl.name)},
    }


# The five problem sizes the method is specified on, in their published order.
CONFIG_WORKLOADS = ("tiny_headwise_f32", "qkv_headwise_bf16", "lowrank_bf16", "alllinear_headwise_bf16",
                    "longseq_lowrank_bf16")


# The short convolutions of the linear-RNN hosts (one filter per channel), timed beside
# the configurations in the default run under the key "hosts".
HOST_WORKLOADS = ("mamba2_xbc_headwise_bf16", "gdn_qkv_headwise_bf16")

# Paths outside the matrix-core and power-of-two head layouts, timed the same way under
# the key "other_paths".
OTHER_WORKLOADS = ("lowrank_f32", "qkv_headwise24_bf16")


def all_configs(a, done: dict, names=CONFIG_WORKLOADS) -> list:
    """Every configuration on the GPU alone (no CPU baseline): the launches of each
    timed the same way as the headline, its own roofline, one record per config."""
    import torch

    from dynamic_short_convolutions_amd.synthetic import WORKLOADS, draw

    out = []
    for i, name in enumerate(names):
        wl = WORKLOADS[name]
        if name in done:
            rec, ms = done[name]
            steps = a.steps
        else:
            print(f"[bench] config {i + 1}: drawing {name}", file=sys.stderr, flush=True)
            inp = draw(wl, need_dy=wl.backward)
            fwd, bwd, kern, keep = training_calls(wl, inp)
            del inp
            m = time_training(fwd, bwd, a.config_steps, a.config_warmup)
            rec = training_record(wl, m, kern)
            ms, steps = m, a.config_steps
            del fwd, bwd, keep
            torch.cuda.empty_cache()
        entry = {"config": i + 1 if names is CONFIG_WORKLOADS else name, "workload": name, "B": wl.B, "T": wl.T,
                 "D": wl.D, "W": wl.W,
                 **({"Hc": wl.Hc} if wl.kind == "headwise" else {"R": wl.R}), "dtype": wl.dtype,
                 "passes": "fwd+bwd" if wl.backward else "fwd",
                 "tokens_per_s": rec["tokens_per_s"], "hbm_GBps": rec["hbm_GBps"],
                 "hbm_frac_of_peak": rec["hbm_frac_of_peak"], "roofline": rec["roofline"]}
        entry["launch_us"] = {k: v * 1e3 for k, v in ms["launch_ms"].items()}
        entry["steps"] = steps
        out.append(entry)
    return out

if __name__ == "__main__":
    sys.exit(main())
