#!/usr/bin/env python3
"""Benchmark of the fused SVDQuant W4A4 linear layer on one MI355X.

One step = one pass of the layer's hot path over one batch: Kernel A
(quantize + down projection) then Kernel B (W4A4 GEMM + up projection + bias),
the same two launches svdq_linear makes, on the FLUX-like fused QKV projection
(M=4608 tokens, K=3072, N=9216, rank 32, int4 group 64) by default.

Inputs are seeded synthetic layers, resident in HBM before timing starts.
Three copies of every input and output buffer are rotated so that a step never
finds its operands in the 256 MB last-level cache (MALL) from the previous
step.  Timing: W warm-up steps, then K timed steps bracketed by device
synchronizations; HIP events on the launch stream give each kernel's average
duration.  Prints one JSON line.

The CPU baseline times the CPU oracle (the layer's plain numpy definition) on
the first rows of the same layer, on this host's cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np

METRIC = "µs and effective TOPS per fused W4A4+rank-32 linear (FLUX shapes); % MFMA peak"
INT8_PEAK_TOPS = 5000.0          # MI355X dense INT8 MFMA, 5.0 POP/s
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, 8 TB/s

WORKLOADS = {
    # name: (M, K, N, r, synth config layer)
    "qkv": (4608, 3072, 9216, 32, "c1_qkv"),
    "fc1": (4608, 3072, 12288, 32, "c2_fc1"),
    "fc2": (4608, 12288, 3072, 32, "c2_fc2"),
}
ROTATE = 3


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default="qkv")
    ap.add_argument("--rank", type=int, default=None, help="override r (0 = bare W4A4 GEMM)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU oracle time")
    ap.add_argument("--variant", choices=["fused", "unfused", "w4a16"], default="fused")
    ap.add_argument("--fmt", choices=["int4_e2m3", "int4"], default="int4_e2m3",
                    help="INT4 g64 codes in the 6-bit E2M3 container (FP6 MFMA) or packed nibbles (INT8 MFMA)")
    return ap.parse_args()


def algorithmic_bytes(M, K, N, r, code_bits=4, G=64):
    """HBM bytes the two kernels must move at minimum (codes at code_bits, fp16 scales / T / Y)."""
    cb = code_bits / 8
    ka = 2 * M * K + 2 * K * r + int(M * K * cb) + 2 * M * K // G + 2 * M * r
    kb = (int(M * K * cb) + 2 * M * K // G + 2 * M * r + int(K * N * cb) + 2 * K * N // G + 2 * r * N + 2 * N
          + 2 * M * N)
    return ka, kb


def cpu_baseline(raw, host_layer, fmt, M, K, N, r, target_s):
    """Time the CPU oracle's per-call work (quantize X, GEMM on the dequantized operands,
    branch, bias, fp16 rounding) on the first rows of the layer."""
    import oracle
    x_hat = host_layer.smooth(raw.x)
    wq, ws, _ = oracle.quant.quantize(host_layer.r_t, fmt)          # offline, not timed
    l1 = np.ascontiguousarray(host_layer.l1t.T)

    def run(m):
        xs = np.ascontiguousarray(x_hat[:m])
        t0 = time.perf_counter()
        q, s, _ = oracle.quant.quantize(xs, fmt)
        t = oracle.forward.down_projection(xs, l1)
        oracle.forward.linear(q, s, t, wq, ws, host_layer.l2, host_layer.bias, fmt)
        return time.perf_counter() - t0

    probe_m = 128
    t_probe = run(probe_m)
    m = int(min(M, max(probe_m, probe_m * target_s / max(t_probe, 1e-3))))
    m = max(probe_m, (m // 64) * 64)
    dt = run(m)
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    tops = 2.0 * m * N * K / dt / 1e12
    return {"value": round(tops, 6), "unit": "TOPS", "cores": int(threads), "kind": "oracle",
            "sample": f"first {m} of {M} token rows of the same layer; one oracle call (quantize X, "
                      f"float64 GEMM on dequantized codes, rank-{r} branch, bias, fp16 rounding) took "
                      f"{dt:.2f} s; value = 2*m*N*K / time",
            "seconds": round(dt, 3)}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU: the layer runs on a single device and this build has no "
              f"multi-GPU path (asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)

    import torch
    from bit_w4a4_quantized_amd import binding
    from bit_w4a4_quantized_amd.prepare import prepare_host, to_device
    from synth import CONFIGS, draw_layer, fc2_calibration_input, LayerShape

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    binding.lib()
    M, K, N, r, lname = WORKLOADS[args.workload]
    fmt = args.fmt
    if args.rank is not None:
        r = args.rank
    shapes = {s.name: s for v in CONFIGS.values() for s in v}
    s = shapes[lname]
    t0 = time.time()
    if lname == "c2_fc2":
        fc1 = draw_layer(shapes["c2_fc1"])
        raw = draw_layer(LayerShape(s.name, s.M, s.K, s.N, r, fmt, s.seed, s.planted_rank))
        raw.x = fc2_calibration_input(fc1)
    else:
        raw = draw_layer(LayerShape(s.name, s.M, s.K, s.N, r, fmt, s.seed, s.planted_rank))
    host = prepare_host(raw.x, raw.w, raw.b, r)
    layer = to_device(host, fmt)
    x_hat = torch.from_numpy(host.smooth(raw.x)).cuda()
    print(f"[bench] prepared {args.workload} M={M} K={K} N={N} r={r} {fmt} in {time.time() - t0:.1f}s",
          file=sys.stderr, flush=True)

    # rotated copies of every operand so that consecutive steps miss in the MALL
    sets = []
    for i in range(ROTATE):
        cp = lambda t: None if t is None else t.clone()
        sets.append(dict(
            x=x_hat.clone(), l1t=cp(layer.l1t), wq=layer.wq.clone(), ws=layer.ws.clone(), l2=cp(layer.l2),
            b=layer.bias.clone(),
            xq=torch.empty(binding.code_shape(M, K, fmt), dtype=torch.uint8, device="cuda"),
            xs=torch.empty(binding.scale_shape(M, K, fmt), dtype=binding.scale_dtype(fmt), device="cuda"),
            t=torch.empty((M, r), dtype=torch.float16, device="cuda") if r else None,
            y=torch.empty((M, N), dtype=torch.float16, device="cuda"),
            ws_buf=torch.empty(max(16, binding.linear_unfused_workspace_bytes(M, N, K, r, fmt)), dtype=torch.uint8, device="cuda"),
        ))
    if args.variant == "w4a16":
        xraw = torch.from_numpy(raw.x).cuda()
        w_t = torch.from_numpy(np.ascontiguousarray(raw.w.T.astype(np.float32))).cuda()
        wq16, ws16 = binding.svdq_quantize_weight(w_t, "int4")
        for st in sets:
            st["xr"], st["wq16"], st["ws16"] = xraw.clone(), wq16.clone(), ws16.clone()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    n_ev = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n_ev)]

    def step(i, record=None):
        st = sets[i % ROTATE]
        if record is not None:
            record[0].record(stream)
        if args.variant == "fused":
            binding.svdq_quantize_down(st["x"], st["l1t"], fmt, xq=st["xq"], xs=st["xs"], t=st["t"])
            if record is not None:
                record[1].record(stream)
            binding.svdq_gemm_w4a4_up(st["xq"], st["xs"], st["t"], st["wq"], st["ws"], st["l2"], st["b"], K, fmt,
                                      y=st["y"])
        elif args.variant == "unfused":
            binding.svdq_linear_unfused(st["x"], st["l1t"], st["wq"], st["ws"], st["l2"], st["b"], fmt,
                                        workspace=st["ws_buf"], y=st["y"])
            if record is not None:
                record[1].record(stream)
        else:
            binding.svdq_gemm_w4a16(st["xr"], st["wq16"], st["ws16"], st["b"], y=st["y"])
            if record is not None:
                record[1].record(stream)
        if record is not None:
            record[2].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(i, ev[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ka_ms = [ev[i][0].elapsed_time(ev[i][1]) for i in range(n_ev)]
    kb_ms = [ev[i][1].elapsed_time(ev[i][2]) for i in range(n_ev)]
    step_ms = [ev[i][0].elapsed_time(ev[i][2]) for i in range(n_ev)]
    ms_per_step = wall * 1e3 / args.steps
    ev_ms = float(np.mean(step_ms))

    # warm-cache figure (same buffers every step), for reference only
    for _ in range(3):
        step(0)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for _ in range(20):
        step(0)
    torch.cuda.synchronize()
    warm_us = (time.perf_counter() - w0) * 1e6 / 20

    ops = 2.0 * M * N * K
    tops = ops / (ms_per_step * 1e-3) / 1e12
    ka_bytes, kb_bytes = algorithmic_bytes(M, K, N, r, 6 if fmt == "int4_e2m3" else 4)
    kb_us = float(np.mean(kb_ms)) * 1e3
    ka_us = float(np.mean(ka_ms)) * 1e3
    if args.variant == "fused":
        dom_ops = ops + 2.0 * M * r * N                       # Kernel B: W4A4 GEMM + up projection
        achieved = dom_ops / (kb_us * 1e-6) / 1e12
        roof = {"kernel": "k_gemm (Kernel B: W4A4 GEMM + up projection)", "bound": "mfma",
                "achieved": round(achieved, 2), "peak": INT8_PEAK_TOPS, "unit": "TFLOP/s",
                "frac": round(achieved / INT8_PEAK_TOPS, 4), "traffic": None,
                "algorithmic": f"2*M*N*K + 2*M*r*N = {dom_ops:.4g} int8-equivalent ops per launch",
                "avg_launch_us": round(kb_us, 2)}
    else:
        roof = {"kernel": args.variant, "bound": "mfma", "achieved": round(tops, 2), "peak": INT8_PEAK_TOPS,
                "unit": "TFLOP/s", "frac": round(tops / INT8_PEAK_TOPS, 4), "traffic": None}

    out = {
        "metric": METRIC,
        "value": round(tops, 3),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4 codes; fp6(e2m3) MFMA" if fmt == "int4_e2m3" else "int4 codes; i8 MFMA",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: {lname} M={M} K={K} N={N} r={r} int4 group 64, fp16 scales",
                   "storage": fmt,
                   "variant": args.variant, "rotated_buffer_sets": ROTATE},
        "us_per_layer": round(ms_per_step * 1e3, 2),
        "us_per_layer_events": round(ev_ms * 1e3, 2),
        "us_per_layer_warm": round(warm_us, 2),
        "pct_int8_peak": round(100.0 * tops / INT8_PEAK_TOPS, 2),
        "kernels_us": {"quantize_down": round(ka_us, 2), "gemm_w4a4_up": round(kb_us, 2)},
        "kernel_a_hbm": {"algorithmic_bytes": ka_bytes,
                         "achieved_GBps": round(ka_bytes / (ka_us * 1e-6) / 1e9, 1) if args.variant == "fused" else None,
                         "frac_of_8TBps": round(ka_bytes / (ka_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4) if args.variant == "fused" else None},
        "roofline": roof,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(raw, host, "int4", M, K, N, r, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
