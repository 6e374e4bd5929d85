#!/usr/bin/env python3
"""Benchmark of the fused SVDQuant W4A4 linear layer on one MI355X.

One step = one pass of the layer's hot path over one batch: Kernel A
(quantize + down projection; K is sliced over workgroups and a small second
launch adds the slices' partial sums of T) then Kernel B (W4A4 GEMM + up
projection + bias), the same launches svdq_linear makes.  The headline line is the FLUX-like
MLP's first linear fc1 (M=4608 tokens, K=3072, N=12288, rank 32, INT4 group 64), the shape
the >= 50%-of-INT8-peak target is stated on; the same run also times, each on its own seeded
layer and with fewer steps:
  * the FLUX-like fused QKV projection (K=3072, N=9216) and the MLP's fc2 (K=12288,
    N=3072), and fc1 on its first 64, 256 and 1024 token rows (small-batch sweep, each point
    against the bound
    its arithmetic intensity puts it under: HBM below 625 op/B, MFMA above; these short
    launches are timed from HIP graph replays, so host launch cost stays out, and the eager
    per-call time is reported beside them);
  * that MLP pair end to end (fc1, GELU + fc2's smoothing, fc2), with the glue as its own
    kernel and with it (and fc1's input smoothing) folded into fc1's two kernels;
  * on the headline layer: the layer with a rank-16 and a rank-32 LoRA adapter carried by its
    branch (rank 48 and 64, same codes), the bare W4A4 GEMM (r = 0: no branch in either kernel),
    the unfused branch (down projection, quantization, GEMM, up projection as
    separate launches with an fp16 intermediate), and the W4A16 control (fp16
    activations times INT4 group-64 weights, no branch) and the fp16 x fp16
    GEMM of the same shape on the vendor library (torch.matmul);
  * the same layer shape in the other code formats: INT8 group 64 (rank 16),
    FP4 E2M1 group 16 with E4M3 scales (rank 32), packed INT4 (rank 32).

Inputs are seeded synthetic layers, resident in HBM before timing starts.
Three copies of every input and output buffer are rotated so that a step never
finds its operands in the 256 MB last-level cache (MALL) from the previous
step.  Timing: untimed steps of the same work for --settle-ms (default 60 ms: the GPU
clock ramps up over the first ~25 ms of sustained load), W warm-up steps, then K timed
steps bracketed by device synchronizations (wall clock); HIP events on the launch stream,
recorded on every 5th timed step (event records add to a step's time), give each kernel's
average duration and the layer's 10/50/90th percentiles.  A shorter run on
one buffer set (operands left in the MALL) gives the warm time beside it.  Prints
one JSON line.

Algorithmic bytes count the method's 4-bit codes (half a byte per code); the bytes the 6-bit
container moves beyond them are reported as their own field.  The roofline's HBM traffic comes
from the committed rocprofv3 counter summary of Kernel B at the same workload (FETCH_SIZE and
WRITE_SIZE, calibrated on a plain copy); it is reported only while Kernel B's sources still
have the hash recorded there.
`--copy-mib N` instead runs the plain copy used for that calibration.

The CPU baseline times the CPU oracle (the layer's plain numpy definition, its GEMM in
float64 on the exactly dequantized operands) on the first rows of the same layer, on this
host's cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np

METRIC = "µs and effective TOPS per fused W4A4+rank-32 linear (FLUX shapes); % MFMA peak"
INT8_PEAK_TOPS = 5000.0          # MI355X dense INT8 MFMA, 5.0 POP/s
FP6_PEAK_TFLOPS = 10100.0        # MI355X dense FP6/FP4 MFMA, 10.1 PFLOP/s
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, 8 TB/s
# Dense matrix-core rates the chip sustains with every SIMD issuing back to back (it then holds
# 1.96 GHz for INT8, 1.9 GHz for FP4, not 2.4): bit_w4a4_quantized_amd/microbench/mfma_clock.hip,
# summarized in profiles/microbench_mfma_clock.md.  Context beside the datasheet peaks above.
INT8_SUSTAINED_TOPS = 3800.0
FP4_SUSTAINED_TFLOPS = 7150.0

WORKLOADS = {
    # name: (M, K, N, r, synthetic layer)
    "qkv": (4608, 3072, 9216, 32, "c1_qkv"),
    "fc1": (4608, 3072, 12288, 32, "c2_fc1"),
    "fc2": (4608, 12288, 3072, 32, "c2_fc2"),
}
ROTATE = 3
COLD_WEIGHT_COPIES = 16                # 16 weight copies: > 256 MB of MALL at fc1's shape
SETTLE_MS = 60.0     # set from --settle-ms
EVENT_EVERY = 5      # HIP events on every 5th timed step: three event records cost ~7 us of a
                     # ~178 us step (measured), so recording them on every step would inflate it


def settle(torch, fn, ms=None):
    """Run fn(i) untimed until at least `ms` of wall time have passed (synchronizing every 8
    calls).  Under sustained load the GPU clock ramps up over the first ~25 ms (per-step times
    of the QKV layer: ~198 us in the first 100 steps, then a flat ~177 us for thousands of
    steps), so every timed measurement starts after such a settle phase."""
    ms = SETTLE_MS if ms is None else ms
    t0, i = time.perf_counter(), 0
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(8):
            fn(i)
            i += 1
        torch.cuda.synchronize()


CSRC = os.path.join(ROOT, "bit_w4a4_quantized_amd", "csrc")
KERNEL_B_SOURCES = {"int4_e2m3": ("k_gemm3.hip",), "int4": ("k_gemm2.hip",),
                    "mxfp4": ("k_gemm_mx.hip", "gemm_skel.h")}


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default="fc1")
    ap.add_argument("--rank", type=int, default=None, help="override r (0 = bare W4A4 GEMM)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="headline only: skip the other workloads "
                                                               "and the bare / unfused / W4A16 comparisons")
    ap.add_argument("--extra-steps", type=int, default=30)
    ap.add_argument("--small-batch-only", action="store_true",
                    help="only the small-batch sweep of the fc1 shape (M = 64, 256, 1024) in --fmt, "
                         "one JSON object (for kernel traces of these launches)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU oracle time")
    ap.add_argument("--settle-ms", type=float, default=60.0,
                    help="untimed steps of the same work for at least this long before each warm-up "
                         "(the GPU clock ramps up over the first ~25 ms of load)")
    ap.add_argument("--fmt", choices=["int4_e2m3", "int4", "mxfp4"], default="int4_e2m3",
                    help="INT4 g64 codes in the 6-bit E2M3 container (FP6 MFMA, the default), packed "
                         "nibbles (INT8 MFMA), or the MXFP4 format (E2M1 g32, E8M0 scales) on the "
                         "block-scaled FP4 MFMA")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="run only a plain device copy of this many MiB (counter calibration)")
    return ap.parse_args()


# scale bytes per element of K: fp16 per 64 (INT4 g64), one E8M0 byte per 32 (MXFP4)
SCALE_BYTES_PER_K = {"int4_e2m3": 2 / 64, "int4": 2 / 64, "mxfp4": 1 / 32}


def algorithmic_bytes(M, K, N, r, fmt="int4"):
    """HBM bytes the two kernels must move at minimum: the method's 4-bit codes (half a byte
    each), the format's scales, fp16 X_hat / T / L1 / L2 / bias / Y."""
    sb = SCALE_BYTES_PER_K[fmt]
    ka = 2 * M * K + 2 * K * r + M * K // 2 + int(M * K * sb) + 2 * M * r
    kb = (M * K // 2 + int(M * K * sb) + 2 * M * r + K * N // 2 + int(K * N * sb) + 2 * r * N + 2 * N
          + 2 * M * N)
    return ka, kb


def container_bytes(M, K, N, fmt):
    """Bytes the storage moves beyond the 4-bit codes: the 6-bit container holds each code in
    three quarters of a byte, so Kernel A writes, and Kernel B reads, M K / 4 more bytes of
    activation codes, and Kernel B reads N K / 4 more of weight codes."""
    if fmt != "int4_e2m3":
        return 0, 0
    return M * K // 4, M * K // 4 + N * K // 4


def kernel_sources_sha256(fmt):
    """One SHA-256 over Kernel B's sources for this format (the files, in order)."""
    h = hashlib.sha256()
    for f in KERNEL_B_SOURCES.get(fmt, ()):
        h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()


def traffic_profile(workload, M, K, N):
    return os.path.join(ROOT, "profiles", f"kernel_b_{workload}_{M}x{K}x{N}_traffic.md")


def kernel_b_traffic(fmt, workload, M, K, N, r):
    """HBM bytes per Kernel B launch from the committed counter summary of this workload, if it
    was taken on the current sources of Kernel B (else None)."""
    path = traffic_profile(workload, M, K, N)
    if fmt != "int4_e2m3" or r != 32 or not os.path.exists(path):
        return None
    m = re.search(r"traffic_json:\s*(\{.*\})", open(path).read())
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("kernel_sources_sha256") != kernel_sources_sha256(fmt):
        return None
    return rec


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
            "gemm_precision": "float64 (the oracle as it stands: exact dequantized operands, "
                              "numpy BLAS dgemm)",
            "seconds": round(dt, 3)}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class Layer:
    """One seeded layer on the device with ROTATE copies of every operand."""

    def __init__(self, torch, binding, name, fmt, r_override=None):
        from bit_w4a4_quantized_amd.prepare import prepare_host, to_device
        from synth import CONFIGS, draw_layer, fc2_calibration_input, LayerShape
        M, K, N, r, lname = WORKLOADS[name]
        if r_override is not None:
            r = r_override
        shapes = {s.name: s for v in CONFIGS.values() for s in v}
        s = shapes[lname]
        t0 = time.time()
        raw = draw_layer(LayerShape(s.name, s.M, s.K, s.N, r, fmt, s.seed, s.planted_rank))
        if lname == "c2_fc2":
            raw.x = fc2_calibration_input(draw_layer(shapes["c2_fc1"]))
        host = prepare_host(raw.x, raw.w, raw.b, r)
        dev = to_device(host, fmt)
        x_hat = torch.from_numpy(host.smooth(raw.x)).cuda()
        self.name, self.lname, self.fmt, self.M, self.K, self.N, self.r = name, lname, fmt, M, K, N, r
        self.raw, self.host, self.torch, self.binding = raw, host, torch, binding
        self.lam = dev.lam                   # fp32 [K], this layer's smoothing factors
        cp = lambda t: None if t is None else t.clone()
        self.sets = []
        for _ in range(ROTATE):
            self.sets.append(dict(
                x=x_hat.clone(), l1t=cp(dev.l1t), wq=dev.wq.clone(), ws=dev.ws.clone(), l2=cp(dev.l2),
                b=dev.bias.clone(),
                xq=torch.empty(binding.code_shape(M, K, fmt), dtype=torch.uint8, device="cuda"),
                xs=torch.empty(binding.scale_shape(M, K, fmt), dtype=binding.scale_dtype(fmt), device="cuda"),
                t=torch.empty((M, r), dtype=torch.float16, device="cuda") if r else None,
                y=torch.empty((M, N), dtype=torch.float16, device="cuda"),
                wsa=torch.empty(max(16, binding.quantize_down_workspace_bytes(M, K, r, fmt)), dtype=torch.uint8,
                                device="cuda"),
            ))
        torch.cuda.synchronize()
        log(f"prepared {name} M={M} K={K} N={N} r={r} {fmt} in {time.time() - t0:.1f}s")

    def fused(self, i, ev=None, branch=True, rotate=ROTATE):
        st, b = self.sets[i % rotate], self.binding
        if ev is not None:
            ev[0].record()
        b.svdq_quantize_down(st["x"], st["l1t"] if branch else None, self.fmt, xq=st["xq"], xs=st["xs"],
                             t=st["t"] if branch else None, workspace=st["wsa"])
        if ev is not None:
            ev[1].record()
        b.svdq_gemm_w4a4_up(st["xq"], st["xs"], st["t"] if branch else None, st["wq"], st["ws"],
                            st["l2"] if branch else None, st["b"], self.K, self.fmt, y=st["y"])
        if ev is not None:
            ev[2].record()

    def time_fused(self, steps, warmup, branch=True, rotate=ROTATE):
        """rotate = ROTATE: operands leave the MALL between steps (cold); rotate = 1: the same
        buffers every step (warm)."""
        torch = self.torch
        ev = {i: [torch.cuda.Event(enable_timing=True) for _ in range(3)] for i in range(0, steps, EVENT_EVERY)}
        settle(torch, lambda i: self.fused(i, branch=branch, rotate=rotate))
        for i in range(warmup):
            self.fused(i, branch=branch, rotate=rotate)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            self.fused(i, ev.get(i), branch=branch, rotate=rotate)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ev = list(ev.values())
        layer = np.array([e[0].elapsed_time(e[2]) for e in ev]) * 1e3
        return {"us_per_layer": wall * 1e6 / steps,
                "us_per_layer_events": float(np.mean(layer)),
                "us_per_layer_events_p10_p50_p90": [round(float(v), 2) for v in np.percentile(layer, [10, 50, 90])],
                "ka_us": float(np.mean([e[0].elapsed_time(e[1]) for e in ev])) * 1e3,
                "kb_us": float(np.mean([e[1].elapsed_time(e[2]) for e in ev])) * 1e3}

    def time_rows_graph(self, m, replays, warmup, calls=2 * ROTATE):
        """The fused layer on the first m token rows, timed from HIP graphs: one graph holds
        `calls` layer calls (rotating buffer sets), another the same Kernel A calls alone, a
        third the Kernel B calls alone, so host launch cost stays out of these small launches.
        After the replays, Y must equal the eager call's Y bit for bit (deterministic kernels)."""
        b, torch = self.binding, self.torch
        K, fmt = self.K, self.fmt
        sets = self._row_sets(m)

        def ka(st):
            b.svdq_quantize_down(st["x"], st["l1t"], fmt, xq=st["xq"], xs=st["xs"], t=st["t"], workspace=st["wsa"])

        def kb(st):
            b.svdq_gemm_w4a4_up(st["xq"], st["xs"], st["t"], st["wq"], st["ws"], st["l2"], st["b"], K, fmt, y=st["y"])
        for st in sets:                      # eager: every set's Kernel B inputs are valid
            ka(st)
            kb(st)
        torch.cuda.synchronize()
        y_eager = sets[0]["y"].clone()
        side = torch.cuda.Stream()
        graphs = {}
        for name, parts in (("layer", (ka, kb)), ("ka", (ka,)), ("kb", (kb,))):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=side):
                for i in range(calls):
                    for fn in parts:
                        fn(sets[i % ROTATE])
            graphs[name] = g
        res = {}
        for name, g in graphs.items():
            settle(torch, lambda i: g.replay())
            for _ in range(warmup):
                g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(replays):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            res[name] = e0.elapsed_time(e1) * 1e3 / (replays * calls)
            if not torch.equal(sets[0]["y"], y_eager):
                raise RuntimeError(f"graph replay ({name}, M={m}) changed Y")
        del graphs
        return {"us_per_layer": res["layer"], "ka_us": res["ka"], "kb_us": res["kb"]}

    def time_rows_graph_cold(self, m, replays, warmup, copies=COLD_WEIGHT_COPIES):
        """As time_rows_graph, but every call of a graph reads its own copy of the weights
        (codes, scales, L2, bias): `copies` copies hold more bytes than the 256 MB MALL, so each
        call streams its weights from HBM, as a layer does when other layers' weights have
        passed through the MALL since its last call.  Returns the layer's and Kernel B's us."""
        b, torch = self.binding, self.torch
        K, fmt = self.K, self.fmt
        sets = self._row_sets(m)
        st0 = self.sets[0]
        wc = [dict(wq=st0["wq"].clone(), ws=st0["ws"].clone(), l2=None if st0["l2"] is None else st0["l2"].clone(),
                   b=st0["b"].clone()) for _ in range(copies)]

        def ka(st):
            b.svdq_quantize_down(st["x"], st["l1t"], fmt, xq=st["xq"], xs=st["xs"], t=st["t"], workspace=st["wsa"])

        def kb(st, w):
            b.svdq_gemm_w4a4_up(st["xq"], st["xs"], st["t"], w["wq"], w["ws"], w["l2"], w["b"], K, fmt, y=st["y"])
        for st in sets:
            ka(st)
            kb(st, wc[0])
        torch.cuda.synchronize()
        y_eager = sets[0]["y"].clone()
        side = torch.cuda.Stream()
        res = {}
        for name, with_a in (("layer", True), ("kb", False)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=side):
                for i in range(copies):
                    if with_a:
                        ka(sets[i % ROTATE])
                    kb(sets[i % ROTATE], wc[i])
            settle(torch, lambda i: g.replay())
            for _ in range(warmup):
                g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(replays):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            res[name] = e0.elapsed_time(e1) * 1e3 / (replays * copies)
            if not torch.equal(sets[0]["y"], y_eager):
                raise RuntimeError(f"cold graph replay ({name}, M={m}) changed Y")
            del g
        del wc
        torch.cuda.empty_cache()
        return {"us_per_layer": res["layer"], "kb_us": res["kb"]}

    def _row_sets(self, m):
        b, torch = self.binding, self.torch
        K, N, r, fmt = self.K, self.N, self.r, self.fmt
        sets = []
        for st in self.sets:
            sets.append(dict(
                x=st["x"][:m], l1t=st["l1t"], wq=st["wq"], ws=st["ws"], l2=st["l2"], b=st["b"],
                xq=torch.empty(b.code_shape(m, K, fmt), dtype=torch.uint8, device="cuda"),
                xs=torch.empty(b.scale_shape(m, K, fmt), dtype=b.scale_dtype(fmt), device="cuda"),
                t=torch.empty((m, r), dtype=torch.float16, device="cuda") if r else None,
                y=torch.empty((m, N), dtype=torch.float16, device="cuda"),
                wsa=torch.empty(max(16, b.quantize_down_workspace_bytes(m, K, r, fmt)), dtype=torch.uint8,
                                device="cuda")))
        return sets

    def time_rows(self, m, steps, warmup):
        """The fused layer on the first m token rows (own code/scale/T/Y buffers, same weights),
        eager calls: what a Python caller sees, host launch cost included."""
        b, torch = self.binding, self.torch
        K, fmt = self.K, self.fmt
        sets = self._row_sets(m)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]

        def one(i, e=None):
            st = sets[i % ROTATE]
            if e is not None:
                e[0].record()
            b.svdq_quantize_down(st["x"], st["l1t"], fmt, xq=st["xq"], xs=st["xs"], t=st["t"], workspace=st["wsa"])
            if e is not None:
                e[1].record()
            b.svdq_gemm_w4a4_up(st["xq"], st["xs"], st["t"], st["wq"], st["ws"], st["l2"], st["b"], K, fmt, y=st["y"])
            if e is not None:
                e[2].record()
        settle(torch, one)
        for i in range(warmup):
            one(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            one(i, ev[i])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return {"us_per_layer": wall * 1e6 / steps,
                "ka_us": float(np.mean([e[0].elapsed_time(e[1]) for e in ev])) * 1e3,
                "kb_us": float(np.mean([e[1].elapsed_time(e[2]) for e in ev])) * 1e3}

    def time_rows_prepared(self, m, steps, warmup):
        """The fused layer on the first m token rows through the prepared-layer binding
        (SvdqLinear: weight side checked once, one svdq_linear call per step): eager calls, host
        launch cost included."""
        b = self.binding
        sets = self._row_sets(m)
        layers = [b.SvdqLinear(st["wq"], st["ws"], st["l1t"], st["l2"], st["b"], self.K, self.fmt) for st in sets]

        def one(i):
            k = i % ROTATE
            layers[k](sets[k]["x"], sets[k]["y"])
        return self.time_call(one, steps, warmup)

    def time_call(self, fn, steps, warmup):
        torch = self.torch
        settle(torch, fn)
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        for i in range(steps):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return {"us_per_call": (time.perf_counter() - t0) * 1e6 / steps,
                "us_per_call_events": e0.elapsed_time(e1) * 1e3 / steps}

    def time_unfused(self, steps, warmup):
        b, torch = self.binding, self.torch
        wsb = torch.empty(max(16, b.linear_unfused_workspace_bytes(self.M, self.N, self.K, self.r, self.fmt)),
                          dtype=torch.uint8, device="cuda")

        def fn(i):
            st = self.sets[i % ROTATE]
            b.svdq_linear_unfused(st["x"], st["l1t"], st["wq"], st["ws"], st["l2"], st["b"], self.fmt,
                                  workspace=wsb, y=st["y"])
        return self.time_call(fn, steps, warmup)

    def time_w4a16(self, steps, warmup):
        b, torch = self.binding, self.torch
        w_t = torch.from_numpy(np.ascontiguousarray(self.raw.w.T.astype(np.float32))).cuda()
        wq16, ws16 = b.svdq_quantize_weight(w_t, "int4")
        del w_t
        xr = [torch.from_numpy(self.raw.x).cuda() for _ in range(ROTATE)]
        wq = [wq16.clone() for _ in range(ROTATE)]
        ws = [ws16.clone() for _ in range(ROTATE)]

        def fn(i):
            st = self.sets[i % ROTATE]
            b.svdq_gemm_w4a16(xr[i % ROTATE], wq[i % ROTATE], ws[i % ROTATE], st["b"], y=st["y"])
        return self.time_call(fn, steps, warmup)


def time_lora(L, steps, warmup):
    """The layer with a LoRA adapter of rank 16 and of rank 32 carried by its branch
    (attach_lora: rank 48 and 64), the residual's codes reused; per-layer time beside the
    plain rank-32 layer's from the same call."""
    from bit_w4a4_quantized_amd.prepare import attach_lora
    torch = L.torch
    g = np.random.default_rng(5)
    res = {"r32_us": round(L.time_fused(steps, warmup)["us_per_layer"], 2)}
    keys = ("l1t", "l2", "t", "wsa")
    saved = [{k: st[k] for k in keys} for st in L.sets]
    for ra in (16, 32):
        a = (g.standard_normal((L.K, ra)) * 0.02).astype(np.float16)
        b = (g.standard_normal((ra, L.N)) * 0.02).astype(np.float16)
        hl = attach_lora(L.host, a, b, 1.0)
        rr = hl.l1t.shape[0]
        for st in L.sets:
            st["l1t"] = torch.from_numpy(hl.l1t).cuda()
            st["l2"] = torch.from_numpy(hl.l2).cuda()
            st["t"] = torch.empty((L.M, rr), dtype=torch.float16, device="cuda")
            st["wsa"] = torch.empty(max(16, L.binding.quantize_down_workspace_bytes(L.M, L.K, rr, L.fmt)),
                                    dtype=torch.uint8, device="cuda")
        t = L.time_fused(steps, warmup)
        res[f"r32_plus_lora{ra}_us"] = round(t["us_per_layer"], 2)
        res[f"r32_plus_lora{ra}_kernels_us"] = {"quantize_down": round(t["ka_us"], 2), "gemm_w4a4_up": round(t["kb_us"], 2)}
    for st, sv in zip(L.sets, saved):
        st.update(sv)
    return res


def time_mlp_pair(fc1, fc2, steps, warmup):
    """The MLP pair fc1 -> GELU + fc2's smoothing -> fc2 (the same layers as the fc1 and fc2
    workloads), with the glue as its own kernel (fc1's input smoothed beforehand on the host,
    so that step is not timed) and with both steps folded into fc1's kernels (Kernel A smooths
    fc1's raw input; Kernel B's epilogue writes fc2's smoothed input).  The two give fc2 the
    same input bit for bit, which is checked."""
    b, torch, fmt = fc1.binding, fc1.torch, fc1.fmt
    x_raw = [torch.from_numpy(fc1.raw.x).cuda() for _ in range(ROTATE)]

    def unfolded(i):
        s1, s2 = fc1.sets[i % ROTATE], fc2.sets[i % ROTATE]
        fc1.fused(i)
        b.svdq_gelu_tanh_smooth(s1["y"], fc2.lam, out=s2["x"])
        fc2.fused(i)

    def folded(i):
        s1, s2 = fc1.sets[i % ROTATE], fc2.sets[i % ROTATE]
        b.svdq_quantize_down_smooth(x_raw[i % ROTATE], fc1.lam, s1["l1t"], fmt, xq=s1["xq"], xs=s1["xs"],
                                    t=s1["t"], workspace=s1["wsa"])
        b.svdq_gemm_w4a4_up_gelu_smooth(s1["xq"], s1["xs"], s1["t"], s1["wq"], s1["ws"], s1["l2"], s1["b"],
                                        fc2.lam, fc1.K, fmt, y=s2["x"])
        fc2.fused(i)

    def glue(i):
        s1, s2 = fc1.sets[i % ROTATE], fc2.sets[i % ROTATE]
        b.svdq_gelu_tanh_smooth(s1["y"], fc2.lam, out=s2["x"])

    unfolded(0)
    torch.cuda.synchronize()
    ref = fc2.sets[0]["x"].clone()
    folded(0)
    torch.cuda.synchronize()
    same = bool(torch.equal(ref.view(torch.int16), fc2.sets[0]["x"].view(torch.int16)))
    tu = fc1.time_call(unfolded, steps, warmup)
    tf = fc1.time_call(folded, steps, warmup)
    tg = fc1.time_call(glue, steps, warmup)
    res = {"unfolded_us": round(tu["us_per_call"], 2), "folded_us": round(tf["us_per_call"], 2),
           "glue_kernel_us": round(tg["us_per_call"], 2),
           "folded_saves_pct": round(100.0 * (1.0 - tf["us_per_call"] / tu["us_per_call"]), 2),
           "fc2_input_bitwise_equal": same,
           "note": "unfolded: svdq_linear(fc1 on X_hat smoothed on the host) + svdq_gelu_tanh_smooth + "
                   "svdq_linear(fc2); folded: svdq_quantize_down_smooth(raw X) + "
                   "svdq_gemm_w4a4_up_gelu_smooth + svdq_linear(fc2)"}
    if not same:
        raise RuntimeError("folded and unfolded MLP pairs gave fc2 different inputs")
    return res


def device_facts(torch):
    """The device and runtime the numbers were taken on."""
    p = torch.cuda.get_device_properties(0)
    facts = {"name": p.name, "arch": getattr(p, "gcnArchName", None), "compute_units": p.multi_processor_count,
             "hbm_gib": round(p.total_memory / 2**30, 1), "torch_hip": torch.version.hip}
    try:
        import ctypes
        lib = os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so")
        hip = ctypes.CDLL(lib if os.path.exists(lib) else "libamdhip64.so")
        v = ctypes.c_int(0)
        if hip.hipDeviceGetAttribute(ctypes.byref(v), 5, 0) == 0:      # hipDeviceAttributeClockRate (kHz)
            facts["peak_clock_mhz"] = v.value // 1000
        if hip.hipRuntimeGetVersion(ctypes.byref(v)) == 0:
            facts["hip_runtime"] = v.value
    except OSError:
        pass
    return facts


def copy_calibration(mib):
    """A plain device copy of known size (for FETCH_SIZE / WRITE_SIZE calibration)."""
    import torch
    n = mib * (1 << 20)
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": n, "launches": 3}), flush=True)


def layer_entry(Lo, res, fmt):
    """Per-layer timing record of a workload other than the headline."""
    o_ops = 2.0 * Lo.M * Lo.N * Lo.K
    o_b = o_ops + 2.0 * Lo.M * Lo.r * Lo.N
    return {"M": Lo.M, "K": Lo.K, "N": Lo.N, "r": Lo.r,
            "us_per_layer": round(res["us_per_layer"], 2),
            "tops": round(o_ops / (res["us_per_layer"] * 1e-6) / 1e12, 2),
            "pct_int8_peak": round(100.0 * o_ops / (res["us_per_layer"] * 1e-6) / 1e12 / INT8_PEAK_TOPS, 2),
            "kernels_us": {"quantize_down": round(res["ka_us"], 2), "gemm_w4a4_up": round(res["kb_us"], 2)},
            "kernel_b_pct_int8_peak": round(100.0 * o_b / (res["kb_us"] * 1e-6) / 1e12 / INT8_PEAK_TOPS, 2)}


def small_batch_sweep(Lo, fmt, es, ew, rows=(64, 256, 1024)):
    """fc1's shape on its first 64, 256 and 1024 token rows: where the layer moves from
    HBM-bound to MFMA-bound (ridge 625 op/B for INT8), timed from HIP graph replays."""
    sweep = {}
    for m in rows:
        rs = Lo.time_rows_graph(m, 20, 3)
        cold = Lo.time_rows_graph_cold(m, 10, 3)
        eager = Lo.time_rows(m, es, ew)
        prepared = Lo.time_rows_prepared(m, es, ew)
        a_b, b_b = algorithmic_bytes(m, Lo.K, Lo.N, Lo.r, fmt)
        c_a, c_b = container_bytes(m, Lo.K, Lo.N, fmt)
        m_ops = 2.0 * m * Lo.N * Lo.K
        layer_s = rs["us_per_layer"] * 1e-6
        intensity = m_ops / (a_b + b_b)
        bound = "hbm" if intensity < INT8_PEAK_TOPS * 1e12 / (HBM_PEAK_GBS * 1e9) else "mfma"
        sweep[str(m)] = {
            "timing": "HIP graph replay",
            "us_per_layer": round(rs["us_per_layer"], 2),
            "us_per_layer_eager_calls": round(eager["us_per_layer"], 2),
            "us_per_layer_eager_prepared_layer": round(prepared["us_per_call"], 2),
            "kernels_us": {"quantize_down": round(rs["ka_us"], 2), "gemm_w4a4_up": round(rs["kb_us"], 2)},
            "us_per_layer_cold_weights": round(cold["us_per_layer"], 2),
            "gemm_w4a4_up_us_cold_weights": round(cold["kb_us"], 2),
            "cold_weights": f"{COLD_WEIGHT_COPIES} weight copies, one per call of the graph (more bytes than the 256 MB MALL)",
            "tops": round(m_ops / layer_s / 1e12, 2),
            "algorithmic_bytes": a_b + b_b,
            "container_extra_bytes": c_a + c_b,
            "ops_per_byte": round(intensity, 1),
            "bound": bound,
            "frac_of_int8_peak": round(m_ops / layer_s / 1e12 / INT8_PEAK_TOPS, 4),
            "frac_of_8TBps": round((a_b + b_b) / layer_s / 1e9 / HBM_PEAK_GBS, 4)}
        log(f"fc1 M={m}: {sweep[str(m)]}")
    return sweep


def main():
    args = parse()
    global SETTLE_MS
    SETTLE_MS = args.settle_ms
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU: the layer runs on a single device and the library has no "
              f"multi-GPU path (asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_mib:
        copy_calibration(args.copy_mib)
        return
    from bit_w4a4_quantized_amd import binding
    binding.lib()
    fmt = args.fmt

    if args.small_batch_only:
        Lo = Layer(torch, binding, "fc1", fmt)
        print(json.dumps({"small_batch_fc1": small_batch_sweep(Lo, fmt, args.extra_steps, 5), "fmt": fmt}),
              flush=True)
        return
    L = Layer(torch, binding, args.workload, fmt, args.rank)
    M, K, N, r = L.M, L.K, L.N, L.r
    head = L.time_fused(args.steps, args.warmup)
    warm = L.time_fused(max(10, args.steps // 4), 3, rotate=1)
    ms_per_step = head["us_per_layer"] * 1e-3

    ops = 2.0 * M * N * K
    tops = ops / (ms_per_step * 1e-3) / 1e12
    ka_bytes, kb_bytes = algorithmic_bytes(M, K, N, r, fmt)
    ka_extra, kb_extra = container_bytes(M, K, N, fmt)
    ka_us, kb_us = head["ka_us"], head["kb_us"]
    dom_ops = ops + 2.0 * M * r * N                       # Kernel B: W4A4 GEMM + up projection
    achieved = dom_ops / (kb_us * 1e-6) / 1e12
    traffic = kernel_b_traffic(fmt, args.workload, M, K, N, r)
    kname = {"int4_e2m3": "k_gemm3", "int4": "k_gemm2", "mxfp4": "k_gemm_mx"}[fmt]
    # a contraction is priced at its own dtype's dense peak: INT8 for the INT4 paths (their
    # integer products), FP4 for MXFP4
    peak = FP6_PEAK_TFLOPS if fmt == "mxfp4" else INT8_PEAK_TOPS
    roof = {"kernel": f"{kname} (Kernel B: W4A4 GEMM + up projection + bias)", "bound": "mfma",
            "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": None if traffic is None else traffic["hbm_bytes_per_launch"],
            "algorithmic": f"2*M*N*K + 2*M*r*N = {dom_ops:.4g} int8-equivalent ops per launch",
            "avg_launch_us": round(kb_us, 2),
            "frac_of_fp6_peak": round(achieved / FP6_PEAK_TFLOPS, 4) if fmt == "int4_e2m3" else None,
            "frac_of_int8_peak": round(achieved / INT8_PEAK_TOPS, 4),
            "frac_of_sustained_mfma_rate": round(achieved / (FP4_SUSTAINED_TFLOPS if fmt == "mxfp4"
                                                             else INT8_SUSTAINED_TOPS), 4),
            "sustained_mfma_rate": {"value": FP4_SUSTAINED_TFLOPS if fmt == "mxfp4" else INT8_SUSTAINED_TOPS,
                                    "source": "profiles/microbench_mfma_clock.md (all SIMDs issuing "
                                              "MFMAs back to back hold 1.9-1.96 GHz)"},
            "algorithmic_hbm_bytes": kb_bytes,
            "container_extra_hbm_bytes": kb_extra}

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
        "dtype": {"int4_e2m3": "int4 codes; fp6(e2m3) MFMA", "int4": "int4 codes; i8 MFMA",
                  "mxfp4": "e2m1 codes, e8m0 scales; block-scaled fp4 MFMA"}[fmt],
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: {L.lname} M={M} K={K} N={N} r={r} "
                               + ("mxfp4 group 32, e8m0 scales" if fmt == "mxfp4" else "int4 group 64, fp16 scales"),
                   "storage": fmt, "rotated_buffer_sets": ROTATE, "settle_ms_before_warmup": SETTLE_MS,
                   "kernel_events_on_every_nth_step": EVENT_EVERY},
        "us_per_layer": round(head["us_per_layer"], 2),
        "us_per_layer_events": round(head["us_per_layer_events"], 2),
        "us_per_layer_events_p10_p50_p90": head["us_per_layer_events_p10_p50_p90"],
        "us_per_layer_warm": round(warm["us_per_layer"], 2),
        "pct_int8_peak": round(100.0 * tops / INT8_PEAK_TOPS, 2),
        "kernels_us": {"quantize_down": round(ka_us, 2), "gemm_w4a4_up": round(kb_us, 2)},
        "kernel_a_hbm": {"algorithmic_bytes": ka_bytes,
                         "container_extra_bytes": ka_extra,
                         "achieved_GBps": round(ka_bytes / (ka_us * 1e-6) / 1e9, 1),
                         "frac_of_8TBps": round(ka_bytes / (ka_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
        "roofline": roof,
        "cpu_baseline": None,
        "device": device_facts(torch),
    }

    if not args.no_extras:
        es, ew = args.extra_steps, 5
        cmp_ = {}
        bare = L.time_fused(es, ew, branch=False)
        fused = L.time_fused(es, ew)
        cmp_["fused_us"] = round(fused["us_per_layer"], 2)
        cmp_["bare_w4a4_us"] = round(bare["us_per_layer"], 2)
        cmp_["bare_kernels_us"] = {"quantize": round(bare["ka_us"], 2), "gemm": round(bare["kb_us"], 2)}
        cmp_["branch_overhead_pct"] = round(100.0 * (fused["us_per_layer"] / bare["us_per_layer"] - 1.0), 2)
        unf = L.time_unfused(es, ew)
        cmp_["unfused_us"] = round(unf["us_per_call"], 2)
        cmp_["unfused_over_fused_pct"] = round(100.0 * (unf["us_per_call"] / fused["us_per_layer"] - 1.0), 2)
        cmp_["unfused_over_bare_pct"] = round(100.0 * (unf["us_per_call"] / bare["us_per_layer"] - 1.0), 2)
        w16 = L.time_w4a16(es, ew)
        cmp_["w4a16_us"] = round(w16["us_per_call"], 2)
        cmp_["speedup_fused_vs_w4a16"] = round(w16["us_per_call"] / fused["us_per_layer"], 3)
        # fp16 x fp16 GEMM of the same shape on the vendor library (torch.matmul -> hipBLASLt)
        xr16 = [torch.from_numpy(L.raw.x).cuda() for _ in range(ROTATE)]
        wt16 = [torch.from_numpy(np.ascontiguousarray(L.raw.w.astype(np.float16))).cuda() for _ in range(ROTATE)]

        def mm(i):
            torch.matmul(xr16[i % ROTATE], wt16[i % ROTATE], out=L.sets[i % ROTATE]["y"])
        cmp_["fp16_gemm_hipblaslt_us"] = round(L.time_call(mm, es, ew)["us_per_call"], 2)
        cmp_["speedup_fused_vs_fp16_hipblaslt"] = round(cmp_["fp16_gemm_hipblaslt_us"] / fused["us_per_layer"], 3)
        cmp_["speedup_w4a16_control_vs_fp16_hipblaslt"] = round(cmp_["fp16_gemm_hipblaslt_us"] / w16["us_per_call"], 3)
        del xr16, wt16
        if L.r == 32:
            cmp_["lora_in_branch"] = time_lora(L, es, ew)
        out["comparisons_" + args.workload] = cmp_
        log(f"comparisons: {cmp_}")
        # the other code formats on the same layer shape (their own rank per setting)
        variants = {}
        for vfmt, vr in (("int8", 16), ("fp4", 32), ("int4", 32), ("mxfp4", 32)):
            Lv = Layer(torch, binding, args.workload, vfmt, vr)
            res = Lv.time_fused(es, ew)
            v_b = ops + 2.0 * M * vr * N
            variants[vfmt] = {"r": vr, "us_per_layer": round(res["us_per_layer"], 2),
                              "tops": round(ops / (res["us_per_layer"] * 1e-6) / 1e12, 2),
                              "kernels_us": {"quantize_down": round(res["ka_us"], 2),
                                             "gemm_w4a4_up": round(res["kb_us"], 2)},
                              "kernel_b_pct_int8_peak": round(100.0 * v_b / (res["kb_us"] * 1e-6) / 1e12 / INT8_PEAK_TOPS, 2),
                              "speedup_vs_w4a16": round(w16["us_per_call"] / res["us_per_layer"], 3)}
            if vfmt == "mxfp4":
                variants[vfmt]["kernel_b_pct_fp4_peak"] = round(
                    100.0 * v_b / (res["kb_us"] * 1e-6) / 1e12 / FP6_PEAK_TFLOPS, 2)
            log(f"variant {vfmt}: {variants[vfmt]}")
            del Lv
            torch.cuda.empty_cache()
        out["formats_" + args.workload] = variants
        others = {}
        layers = {args.workload: L} if args.rank is None else {}
        for name in ("fc1", "qkv", "fc2"):
            if name == args.workload and args.rank is None:
                continue
            Lo = Layer(torch, binding, name, fmt)
            layers[name] = Lo
            others[name] = layer_entry(Lo, Lo.time_fused(es, ew), fmt)
            log(f"{name}: {others[name]}")
        out["other_workloads"] = others
        out["small_batch_fc1"] = small_batch_sweep(layers["fc1"], fmt, es, ew)
        if fmt != "int4":
            # few token rows read mostly weights: the packed layout moves 2/3 of the container's
            # weight bytes (its own weight-streaming kernel, INT8 matrix cores)
            Lp = Layer(torch, binding, "fc1", "int4")
            out["small_batch_fc1_packed_int4"] = small_batch_sweep(Lp, "int4", es, ew, rows=(64, 256))
            del Lp
            torch.cuda.empty_cache()
        pair = time_mlp_pair(layers["fc1"], layers["fc2"], es, ew)
        log(f"mlp pair: {pair}")
        out["mlp_pair_fc1_fc2"] = pair
        del layers
        torch.cuda.empty_cache()

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(L.raw, L.host, "int4", M, K, N, r, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
