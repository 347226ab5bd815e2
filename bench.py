"""Benchmark of the FP8 quantize-then-scaled-GEMM hot path on one MI355X.

One step runs every scaling scheme's full path on its workload, with all inputs resident in HBM:
  per-tensor current   A 16x32, B 32x64 fp32: amax + cast (B transposed), GEMM, fp32 out
  delayed              one of 16 steps of A 1024x2048, B 2048x1024 bf16: casts with fused amax,
                       GEMM (bf16 out), then both amax-history updates
  fine-grained         X 4096x7168 (1x128) and W 2048x7168 (128x128) casts, block-scaled GEMM
  MXFP8                A, B 8192x8192 casts, E8M0-scaled GEMM
  MOSS fwd+bwd         X 16384x4096, W 4096x4096 (E4M3), dY 16384x4096 (E5M2): amax, then one
                       dual-axis cast per tensor (both quantized copies in one pass),
                       Y = X W^T, dX = dY W, dW = dY^T X
After the timed steps, the next-step paths are timed on the same inputs (reported under
"next_rows", not part of the headline): automatic weight scaling against a just-in-time max
reduction of W, the delayed-scaling history merge, UE8M0 128x128 weight quantization and block
dequantization, and the block GEMM with UE8M0 weight scales and with a static activation scale.
Each cast is also timed alone, cold (input from HBM) and warm ("quantize_cold_warm"), beside a
plain 256 MiB device copy timed the same way as the reference for what HBM delivers to a streaming
kernel.
The headline value is the step's total GEMM flops (2 M N K per GEMM) divided by the step time,
i.e. scaled-GEMM TFLOP/s including every quantization the path performs.  "per_config" gives each
workload's GEMM flops over the summed time of all its launches beside the ceiling the two
rooflines allow (GEMM flops at the FP8 MFMA peak plus its cast bytes at the HBM peak).  The
oracle leg ("cpu_baseline", skipped with --no-cpu-baseline) times the CPU oracle per workload on a
bounded sample and, outside that timing, reports the quantization SNR ("snr_db") of the
fine-grained, MX and MOSS operands the timed steps wrote.

The timed steps are replays of HIP graphs captured from the same library calls (one graph per
delayed-scaling step index, since that input changes with the step); --no-graph times eager
launches instead.  Per-kernel times and the roofline come from a second pass of K eager steps with
HIP events around each launch, whose step time is reported as ms_per_step_eager.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-graph]
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

PEAK_FP8_TFLOPS = 5033.0      # MI355X dense FP8 MFMA (256 CU x 8192 flop/clk x 2.4 GHz)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
MOSS_ELEMS = 2 * 16384 * 4096 + 4096 * 4096   # X, dY and W elements
METRIC = "scaled FP8 GEMM TFLOP/s incl. quantize (% FP8 MFMA peak); quantize GB/s"
WORKLOAD = ("all five scaling schemes per step: per-tensor current 16x32x64 fp32, delayed 1024x2048x1024 "
            "bf16, fine-grained 1x128/128x128 4096x7168x2048, MXFP8 8192^3, MOSS fwd+bwd 16384x4096x4096")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="time the steps as eager launches instead of HIP graph replays")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed steps, run one plain 256 MiB device copy (read + write) whose "
                         "known size calibrates the HBM byte counters of a profiler run")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                            "gemm_moss_16384x4096x4096_hbm_traffic.md")
GEMM_SOURCES = ("fp8_scaled_quantization_amd/csrc/gemm_pp.cuh", "fp8_scaled_quantization_amd/csrc/gemm_ppb.cuh",
                "fp8_scaled_quantization_amd/csrc/gemm_pps.cuh",
                "fp8_scaled_quantization_amd/csrc/gemm_kernel.cuh",
                "fp8_scaled_quantization_amd/csrc/gemm.hip", "fp8_scaled_quantization_amd/csrc/kernels.h",
                "fp8_scaled_quantization_amd/csrc/common.cuh")


def _code_only(text):
    """C++ source with its comments removed and whitespace runs collapsed (string and character
    literals kept), so that the digest below changes with the code, not with its comments."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def gemm_source_digest():
    """SHA-256 over the GEMM sources' code (comments and layout excluded)."""
    import hashlib
    h = hashlib.sha256()
    root = os.path.dirname(os.path.abspath(__file__))
    for rel in GEMM_SOURCES:
        with open(os.path.join(root, rel), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch of the MOSS GEMM from the committed counter summary, or None when that
    summary is missing or was taken on GEMM sources other than the ones in this tree."""
    try:
        with open(TRAFFIC_FILE) as f:
            txt = f.read()
    except OSError:
        return None
    fields = dict(line.split(":", 1) for line in txt.splitlines() if line.startswith(("source_sha256:", "bytes_per_launch:")))
    if fields.get("source_sha256", "").strip() != gemm_source_digest():
        return None
    try:
        return int(fields["bytes_per_launch"].strip())
    except (KeyError, ValueError):
        return None


class Timer:
    """HIP events recorded on the stream the library launches on (torch's current stream)."""

    def __init__(self, torch):
        self.torch = torch
        self.events = {}     # name -> list of (start, end)
        self.enabled = False

    def __call__(self, name, fn):
        if not self.enabled:
            fn()
            return
        s = self.torch.cuda.Event(enable_timing=True)
        e = self.torch.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        self.events.setdefault(name, []).append((s, e))

    def mean_ms(self, name):
        ev = self.events.get(name, [])
        return sum(s.elapsed_time(e) for s, e in ev) / max(len(ev), 1)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import fp8_scaled_quantization_amd as fq
    from fp8_scaled_quantization_amd import workloads as wl

    fq.init()
    dev = "cuda:0"
    E4M3, E5M2 = fq.E4M3, fq.E5M2
    TENSOR, BLOCK, MX, MOSS = fq.TENSOR, fq.BLOCK, fq.MX, fq.MOSS

    def dbf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    def zeros(shape, dt):
        return torch.zeros(shape, dtype=dt, device=dev)

    u8, f32, bf16 = torch.uint8, torch.float32, torch.bfloat16
    t0 = time.time()
    # ---------------- inputs (seeded, synthetic), resident in HBM
    a1, b1 = wl.per_tensor_inputs()
    w1 = dict(A=torch.from_numpy(a1).to(dev), B=torch.from_numpy(b1).to(dev))
    w2 = dict(A=[], B=[])
    for t in range(16):
        A, B, _ = wl.delayed_inputs(t)
        w2["A"].append(dbf16(A))
        w2["B"].append(dbf16(B))
    X3, W3 = wl.fine_grained_inputs()
    w3 = dict(X=dbf16(X3), W=dbf16(W3))
    A4, B4 = wl.mx_inputs()
    w4 = dict(A=dbf16(A4), B=dbf16(B4))
    X5, W5, G5 = wl.moss_inputs()
    w5 = dict(X=dbf16(X5), W=dbf16(W5), G=dbf16(G5))
    A2h, B2h, _ = wl.delayed_inputs(0)
    host_inputs = dict(a1=a1, b1=b1, A2=A2h, B2=B2h, X3=X3, W3=W3, A4=A4, B4=B4, X5=X5, W5=W5, G5=G5)
    gen_s = time.time() - t0

    # ---------------- outputs and state, allocated once (the library never allocates)
    o = {}
    o["q1a"], o["q1b"] = zeros((16, 32), u8), zeros((64, 32), u8)
    o["s1a"], o["s1b"], o["m1a"], o["m1b"] = (zeros(1, f32) for _ in range(4))
    o["C1"] = zeros((16, 64), f32)
    o["q2a"], o["q2b"] = zeros((1024, 2048), u8), zeros((1024, 2048), u8)
    o["s2a"], o["s2b"] = torch.ones(1, dtype=f32, device=dev), torch.ones(1, dtype=f32, device=dev)
    o["h2a"], o["h2b"] = zeros(1024, f32), zeros(1024, f32)
    o["m2a"], o["m2b"] = zeros(1, f32), zeros(1, f32)
    o["C2"] = zeros((1024, 1024), bf16)
    o["q3x"], o["s3x"] = zeros((4096, 7168), u8), zeros((4096, 56), f32)
    o["q3w"], o["s3w"] = zeros((2048, 7168), u8), zeros((16, 56), f32)
    o["C3"] = zeros((4096, 2048), bf16)
    o["q4a"], o["e4a"] = zeros((8192, 8192), u8), zeros((8192, 256), u8)
    o["q4b"], o["e4b"] = zeros((8192, 8192), u8), zeros((8192, 256), u8)
    o["C4"] = zeros((8192, 8192), bf16)
    for n, (r, c) in dict(X=(16384, 4096), W=(4096, 4096), G=(16384, 4096)).items():
        o["q5" + n], o["e5" + n] = zeros((r, c), u8), zeros((r, c // 32), u8)
        o["q5" + n + "T"], o["e5" + n + "T"] = zeros((c, r), u8), zeros((c, r // 32), u8)
        o["S5" + n], o["m5" + n] = zeros(1, f32), zeros(1, f32)
    o["Y5"], o["dX5"], o["dW5"] = zeros((16384, 4096), bf16), zeros((16384, 4096), bf16), zeros((4096, 4096), bf16)

    timer = Timer(torch)
    Q, QD, G_ = fq.fp8_quantize, fq.fp8_quantize_dual, fq.fp8_scaled_gemm

    def step(i):
        # per-tensor current scaling
        timer("q1", lambda: (Q(TENSOR, E4M3, w1["A"], o["q1a"], None, o["s1a"], False, o["m1a"]),
                             Q(TENSOR, E4M3, w1["B"], o["q1b"], None, o["s1b"], False, o["m1b"], transpose_out=True)))
        timer("g1", lambda: G_(TENSOR, o["q1a"], E4M3, None, o["q1b"], E4M3, None, o["s1a"], o["s1b"], o["C1"], fq.OUT_F32))
        # delayed scaling: casts with the state's scales (fused amax), GEMM, then history updates
        t = i % 16
        timer("q2", lambda: (Q(TENSOR, E4M3, w2["A"][t], o["q2a"], None, o["s2a"], True, o["m2a"]),
                             Q(TENSOR, E4M3, w2["B"][t], o["q2b"], None, o["s2b"], True, o["m2b"], transpose_out=True)))
        timer("g2", lambda: G_(TENSOR, o["q2a"], E4M3, None, o["q2b"], E4M3, None, o["s2a"], o["s2b"], o["C2"], fq.OUT_BF16))
        timer("h2", lambda: (fq.fp8_history_update(o["h2a"], o["m2a"], o["s2a"], E4M3),
                             fq.fp8_history_update(o["h2b"], o["m2b"], o["s2b"], E4M3)))
        # fine-grained block scaling
        timer("q3x", lambda: Q(BLOCK, E4M3, w3["X"], o["q3x"], o["s3x"], block=(1, 128)))
        timer("q3w", lambda: Q(BLOCK, E4M3, w3["W"], o["q3w"], o["s3w"], block=(128, 128)))
        timer("g3", lambda: G_(BLOCK, o["q3x"], E4M3, o["s3x"], o["q3w"], E4M3, o["s3w"], None, None, o["C3"], fq.OUT_BF16))
        # MXFP8
        timer("q4", lambda: (Q(MX, E4M3, w4["A"], o["q4a"], o["e4a"]), Q(MX, E4M3, w4["B"], o["q4b"], o["e4b"])))
        timer("g4", lambda: G_(MX, o["q4a"], E4M3, o["e4a"], o["q4b"], E4M3, o["e4b"], None, None, o["C4"], fq.OUT_BF16))
        # MOSS forward + backward
        for n, fmt in (("X", E4M3), ("W", E4M3), ("G", E5M2)):
            timer("q5", lambda: QD(MOSS, fmt, w5[n], o["q5" + n], o["e5" + n], o["q5" + n + "T"], o["e5" + n + "T"],
                                   o["S5" + n], False, o["m5" + n]))
        timer("g5", lambda: G_(MOSS, o["q5X"], E4M3, o["e5X"], o["q5W"], E4M3, o["e5W"], o["S5X"], o["S5W"], o["Y5"], fq.OUT_BF16))
        timer("g5", lambda: G_(MOSS, o["q5G"], E5M2, o["e5G"], o["q5WT"], E4M3, o["e5WT"], o["S5G"], o["S5W"], o["dX5"], fq.OUT_BF16))
        timer("g5", lambda: G_(MOSS, o["q5GT"], E5M2, o["e5GT"], o["q5XT"], E4M3, o["e5XT"], o["S5G"], o["S5X"], o["dW5"], fq.OUT_BF16))

    # ---------------- flops and algorithmic bytes
    gemm_flops = {"g1": 2 * 16 * 64 * 32, "g2": 2 * 1024 * 1024 * 2048, "g3": 2 * 4096 * 2048 * 7168,
                  "g4": 2 * 8192 ** 3, "g5": 2 * 16384 * 4096 * 4096}            # g5: per launch
    launches = {"g1": 1, "g2": 1, "g3": 1, "g4": 1, "g5": 3}
    step_flops = sum(gemm_flops[k] * launches[k] for k in gemm_flops)
    # bytes per quantize call: input read (+ the amax pass's read when the scale is derived),
    # FP8 write, scale write
    qbytes = {
        "q1": (16 * 32 + 32 * 64) * 4 * 2 + (16 * 32 + 32 * 64),
        "q2": 2 * (1024 * 2048 * 3),
        "q3x": 4096 * 7168 * 3 + 4096 * 56 * 4,
        "q3w": 2048 * 7168 * 3 + 16 * 56 * 4,
        "q4": 2 * (8192 * 8192 * 3 + 8192 * 256),
        "q5": MOSS_ELEMS * (2 + 2 + 1 + 1) + 2 * (MOSS_ELEMS // 32),     # amax read + one read, two copies
    }
    qcalls = {"q1": 1, "q2": 1, "q3x": 1, "q3w": 1, "q4": 1, "q5": 3}

    # ---------------- warmup, then the timed steps
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    def timed_steps(run):
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for i in range(args.steps):
            run(args.warmup + i)
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end) / args.steps

    graph_ms = None
    if not args.no_graph:
        # One graph per delayed-scaling input index (the step's only varying argument); the library
        # launches on torch's current stream, which is the capture stream inside the block.  Replays
        # advance the delayed-scaling state exactly as eager steps do.
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        graphs = []
        for t in range(16):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=side):
                step(t)
            graphs.append(g)
        torch.cuda.synchronize()
        for i in range(args.warmup):
            graphs[i % 16].replay()
        graph_ms = timed_steps(lambda i: graphs[i % 16].replay())
    # eager steps with per-launch events: the per-kernel times and the roofline
    timer.enabled = True
    eager_ms = timed_steps(step)
    ms_per_step = graph_ms if graph_ms is not None else eager_ms
    tflops = step_flops / (ms_per_step * 1e-3) / 1e12

    per = {}
    for k in gemm_flops:
        ms = timer.mean_ms(k)
        per[k] = dict(ms=round(ms, 5), tflops=round(gemm_flops[k] / (ms * 1e-3) / 1e12, 2),
                      pct_fp8_peak=round(100 * gemm_flops[k] / (ms * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 2))
    for k in qbytes:
        ms = timer.mean_ms(k)
        per_call = qbytes[k] / qcalls[k]
        per[k] = dict(ms=round(ms, 5), gbs=round(per_call / (ms * 1e-3) / 1e9, 1),
                      pct_hbm_peak=round(100 * per_call / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 2))
    per["h2"] = dict(ms=round(timer.mean_ms("h2"), 5))
    quant_ms = sum(timer.mean_ms(k) * qcalls[k] for k in qbytes)
    quant_gbs = sum(qbytes.values()) / (quant_ms * 1e-3) / 1e9
    # each workload's GEMM flops over the time of all of its launches (casts, state updates,
    # GEMMs), beside the ceiling both rooflines allow: flops / (flops / MFMA peak + cast bytes / HBM peak)
    configs = {"per-tensor 16x32x64": (["q1"], ["g1"], []), "delayed 1024x2048x1024": (["q2"], ["g2"], ["h2"]),
               "fine-grained 4096x7168x2048": (["q3x", "q3w"], ["g3"], []),
               "MXFP8 8192^3": (["q4"], ["g4"], []), "MOSS fwd+bwd 16384x4096x4096": (["q5"], ["g5"], [])}
    per_config = {}
    for name, (qs, gs, extra) in configs.items():
        fl = sum(gemm_flops[k] * launches[k] for k in gs)
        ms = sum(timer.mean_ms(k) * qcalls[k] for k in qs) + sum(timer.mean_ms(k) * launches[k] for k in gs) + \
            sum(timer.mean_ms(k) for k in extra)
        by = sum(qbytes[k] for k in qs)
        ideal_s = fl / (PEAK_FP8_TFLOPS * 1e12) + by / (PEAK_HBM_GBS * 1e9)
        per_config[name] = {"ms": round(ms, 5), "tflops_incl_quantize": round(fl / (ms * 1e-3) / 1e12, 2),
                            "pct_fp8_peak": round(100 * fl / (ms * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 2),
                            "ceiling_pct_fp8_peak": round(100 * fl / ideal_s / 1e12 / PEAK_FP8_TFLOPS, 2)}
    w_only = timer.mean_ms("q3x") + timer.mean_ms("g3")
    per_config["fine-grained 4096x7168x2048"]["weights_prequantized"] = {
        "ms": round(w_only, 5), "tflops_incl_quantize": round(gemm_flops["g3"] / (w_only * 1e-3) / 1e12, 2),
        "ceiling_pct_fp8_peak": round(100 * gemm_flops["g3"] / (gemm_flops["g3"] / (PEAK_FP8_TFLOPS * 1e12) +
                                                                 qbytes["q3x"] / (PEAK_HBM_GBS * 1e9)) / 1e12 /
                                      PEAK_FP8_TFLOPS, 2)}
    # dominant kernel: the GEMM launch with the largest total time per step
    dom = max(gemm_flops, key=lambda k: timer.mean_ms(k) * launches[k])
    dom_ms = timer.mean_ms(dom)
    dom_tf = gemm_flops[dom] / (dom_ms * 1e-3) / 1e12
    names = {"g1": "per-tensor GEMM 16x64x32", "g2": "delayed GEMM 1024x1024x2048", "g3": "block GEMM 4096x2048x7168",
             "g4": "MX GEMM 8192x8192x8192", "g5": "MOSS GEMM 16384x4096x4096 (avg of Y, dX, dW)"}
    roofline = {"kernel": names[dom], "bound": "mfma", "achieved": round(dom_tf, 2), "peak": PEAK_FP8_TFLOPS,
                "unit": "TFLOP/s", "frac": round(dom_tf / PEAK_FP8_TFLOPS, 4),
                "traffic": measured_traffic() if dom == "g5" else None, "traffic_unit": "bytes per launch",
                "avg_launch_ms": round(dom_ms, 5)}
    next_rows = measure_next(torch, fq, o, w3, w5, args.steps)
    cold_warm = measure_casts_cold_warm(torch, fq, o, w2, w3, w4, w5)
    if args.copy_calibration:
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)          # 256 MiB read + 256 MiB written
        torch.cuda.synchronize()
        del src, dst

    out = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8 e4m3/e5m2 operands, fp32 accumulate", "data": "synthetic (seeded numpy PCG64)",
        "config": {"workload": WORKLOAD, "gemm_tflop_per_step": round(step_flops / 1e12, 4), "parallelism": "single GPU",
                   "launch": "eager" if graph_ms is None else "HIP graph replay, one graph per delayed-scaling step"},
        "ms_per_step_eager": round(eager_ms, 4),
        "pct_fp8_peak": round(100 * tflops / PEAK_FP8_TFLOPS, 2),
        "quantize_gbs": round(quant_gbs, 1), "quantize_pct_hbm_peak": round(100 * quant_gbs / PEAK_HBM_GBS, 2),
        "roofline": roofline, "per_config": per_config, "per_kernel": per, "quantize_cold_warm": cold_warm,
        "next_rows": next_rows,
        "input_gen_s": round(gen_s, 1),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"], out["snr_db"] = oracle_leg(host_inputs, o, torch)
    print(json.dumps(out), flush=True)


def measure_casts_cold_warm(torch, fq, o, w2, w3, w4, w5, reps=20, warmup=5):
    """Each cast of the step timed alone (HIP events around it), cold and warm: after `warmup`
    untimed launches, the median of `reps` cold launches and the mean of `reps` warm ones.  Cold:
    before every launch a 1 GiB buffer is read, which leaves only clean, unrelated lines in L2 and
    the 256 MB last-level cache, so the input comes from HBM and no earlier writes are pending.  Warm: the
    same launch repeated back to back, so an input that fits the last-level cache is served from
    it.  GB/s counts the algorithmic bytes (input read, plus the amax pass's read where the scale
    is derived, FP8 and scale bytes written).  A plain device copy (256 MiB read, 256 MiB written,
    torch's elementwise kernel) is timed the same way as the reference for what HBM delivers to a
    streaming kernel, and each cast's cold rate is also given as a fraction of the copy's."""
    dev = "cuda:0"
    E4M3, E5M2 = fq.E4M3, fq.E5M2
    TENSOR, BLOCK, MX, MOSS = fq.TENSOR, fq.BLOCK, fq.MX, fq.MOSS
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    sink = torch.zeros(1, dtype=torch.float32, device=dev)
    Q, QD = fq.fp8_quantize, fq.fp8_quantize_dual
    casts = {
        "delayed A 1024x2048 (fused amax)": (lambda: Q(TENSOR, E4M3, w2["A"][0], o["q2a"], None, o["s2a"], True, o["m2a"]),
                                             1024 * 2048 * 3),
        "1x128 X 4096x7168": (lambda: Q(BLOCK, E4M3, w3["X"], o["q3x"], o["s3x"], block=(1, 128)),
                              4096 * 7168 * 3 + 4096 * 56 * 4),
        "128x128 W 2048x7168": (lambda: Q(BLOCK, E4M3, w3["W"], o["q3w"], o["s3w"], block=(128, 128)),
                                2048 * 7168 * 3 + 16 * 56 * 4),
        "MX A 8192x8192": (lambda: Q(MX, E4M3, w4["A"], o["q4a"], o["e4a"]), 8192 * 8192 * 3 + 8192 * 256),
        "MOSS X 16384x4096 (amax + dual cast)": (
            lambda: QD(MOSS, E4M3, w5["X"], o["q5X"], o["e5X"], o["q5XT"], o["e5XT"], o["S5X"], False, o["m5X"]),
            16384 * 4096 * 6 + 2 * 16384 * 128),
    }
    csrc = torch.ones(64 << 20, dtype=torch.float32, device=dev)
    cdst = torch.empty_like(csrc)
    casts["device copy 256 MiB (reference)"] = (lambda: torch.neg(csrc, out=cdst), 2 * csrc.numel() * 4)
    out = {}
    for name, (fn, nbytes) in casts.items():
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        cold = []
        for _ in range(reps):
            torch.sum(flush, dim=0, keepdim=True, out=sink)
            s = torch.cuda.Event(enable_timing=True)
            e = torch.cuda.Event(enable_timing=True)
            s.record()
            fn()
            e.record()
            cold.append((s, e))
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(reps):
            fn()
        e.record()
        torch.cuda.synchronize()
        cold_ms = sorted(a.elapsed_time(b) for a, b in cold)[reps // 2]
        warm_ms = s.elapsed_time(e) / reps
        out[name] = {"cold_ms": round(cold_ms, 5), "cold_gbs": round(nbytes / (cold_ms * 1e-3) / 1e9, 1),
                     "cold_pct_hbm_peak": round(100 * nbytes / (cold_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 2),
                     "warm_ms": round(warm_ms, 5), "warm_gbs": round(nbytes / (warm_ms * 1e-3) / 1e9, 1)}
    del flush, csrc, cdst
    copy = out["device copy 256 MiB (reference)"]["cold_gbs"]
    for v in out.values():
        v["cold_pct_of_copy"] = round(100 * v["cold_gbs"] / copy, 1)
    return out


def measure_next(torch, fq, o, w3, w5, reps):
    """Event-timed averages (reps launches each, after one warm-up) of the next-step paths."""
    dev = "cuda:0"
    E4M3 = fq.E4M3
    BLOCK, BLOCK_E8M0, TENSOR = fq.BLOCK, fq.BLOCK_E8M0, fq.TENSOR

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(reps):
            fn()
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / reps

    def graph_timed(fn, n=50, replays=10):
        """Device time per call: n calls captured in one HIP graph, replayed back to back, so that
        no host launch cost is included (what remains per call is the kernel and its dispatch)."""
        fn()
        torch.cuda.synchronize()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            for _ in range(n):
                fn()
        g.replay()
        torch.cuda.synchronize()
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(replays):
            g.replay()
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / (replays * n)

    W5, W3, X3 = w5["W"], w3["W"], w3["X"]
    amax = torch.zeros(1, dtype=torch.float32, device=dev)
    state = torch.zeros(2, dtype=torch.float32, device=dev)
    sc = torch.zeros(1, dtype=torch.float32, device=dev)
    fq.fp8_amax(W5, amax)
    fq.fp8_auto_scale(state, True, amax, 1e-4, E4M3, sc)
    jit_fn = lambda: (fq.fp8_amax(W5, amax), fq.fp8_auto_scale(state, True, amax, 1e-4, E4M3, sc))
    auto_fn = lambda: fq.fp8_auto_scale(state, False, None, 1e-4, E4M3, sc)
    jit_ms = timed(jit_fn)
    auto_ms = timed(auto_fn)
    jit_dev_ms = graph_timed(jit_fn)
    auto_dev_ms = graph_timed(auto_fn)
    h1 = torch.zeros(1024, dtype=torch.float32, device=dev)
    h2 = torch.rand(1024, dtype=torch.float32, device=dev)
    s1, s2 = torch.ones(1, device=dev), torch.ones(1, device=dev)
    merge_ms = timed(lambda: fq.fp8_history_merge(h1, h2, s1, s2))
    qw8 = torch.empty((2048, 7168), dtype=torch.uint8, device=dev)
    ew8 = torch.empty((16, 56), dtype=torch.uint8, device=dev)
    qe_ms = timed(lambda: fq.fp8_quantize(BLOCK_E8M0, E4M3, W3, qw8, ew8, block=(128, 128)))
    wbf = torch.empty((2048, 7168), dtype=torch.bfloat16, device=dev)
    dq_ms = timed(lambda: fq.fp8_block_dequantize(BLOCK_E8M0, E4M3, qw8, ew8, wbf))
    C = o["C3"]
    g8_ms = timed(lambda: fq.fp8_scaled_gemm(BLOCK_E8M0, o["q3x"], E4M3, o["s3x"], qw8, E4M3, ew8, None, None, C,
                                             fq.OUT_BF16))
    sa = torch.full((1,), float(X3.float().abs().max()) / 448.0, dtype=torch.float32, device=dev)
    qxs = torch.empty((4096, 7168), dtype=torch.uint8, device=dev)
    fq.fp8_quantize(TENSOR, E4M3, X3, qxs, None, sa, True)
    gs_ms = timed(lambda: fq.fp8_scaled_gemm(BLOCK, qxs, E4M3, None, o["q3w"], E4M3, o["s3w"], sa, None, C,
                                             fq.OUT_BF16))
    flops = 2 * 4096 * 2048 * 7168
    wbytes_q = 2048 * 7168 * 3 + 16 * 56
    wbytes_dq = 2048 * 7168 * 3 + 16 * 56
    return {
        "auto_scale_us": round(auto_ms * 1e3, 2),
        "jit_amax_plus_scale_us": round(jit_ms * 1e3, 2),
        "auto_scale_us_device": round(auto_dev_ms * 1e3, 2),
        "jit_amax_plus_scale_us_device": round(jit_dev_ms * 1e3, 2),
        "timing": "*_us: back-to-back eager launches (host launch rate); *_us_device: 50 calls in one HIP graph, "
                  "replayed (device time per call)",
        "jit_tensor": "MOSS W 4096x4096 bf16",
        "history_merge_1024_us": round(merge_ms * 1e3, 2),
        "ue8m0_quantize_w_2048x7168": {"ms": round(qe_ms, 5), "gbs": round(wbytes_q / (qe_ms * 1e-3) / 1e9, 1),
                                       "pct_hbm_peak": round(100 * wbytes_q / (qe_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 2)},
        "block_dequantize_ue8m0_to_bf16_2048x7168": {"ms": round(dq_ms, 5),
                                                     "gbs": round(wbytes_dq / (dq_ms * 1e-3) / 1e9, 1),
                                                     "pct_hbm_peak": round(100 * wbytes_dq / (dq_ms * 1e-3) / 1e9 /
                                                                           PEAK_HBM_GBS, 2)},
        "gemm_block_ue8m0_weights_4096x2048x7168": {"ms": round(g8_ms, 5),
                                                    "tflops": round(flops / (g8_ms * 1e-3) / 1e12, 2),
                                                    "pct_fp8_peak": round(100 * flops / (g8_ms * 1e-3) / 1e12 /
                                                                          PEAK_FP8_TFLOPS, 2)},
        "gemm_block_static_activation_4096x2048x7168": {"ms": round(gs_ms, 5),
                                                        "tflops": round(flops / (gs_ms * 1e-3) / 1e12, 2),
                                                        "pct_fp8_peak": round(100 * flops / (gs_ms * 1e-3) / 1e12 /
                                                                              PEAK_FP8_TFLOPS, 2)},
    }


def oracle_leg(h, o, torch):
    """The CPU oracle timed on the host's cores over a bounded sample of each workload (its
    quantization of sampled rows, or of the whole tensor where small, and its fp64 GEMM over the
    sampled rows and columns), per workload and in total, in the metric's unit (GEMM TFLOP/s incl.
    quantize); then, outside that timing, the quantization SNR of the step's own GPU output (the
    MX and MOSS operands the timed steps wrote), dequantized exactly by the oracle."""
    import oracle.oracle as orc
    from fp8_scaled_quantization_amd import workloads as wl
    lib = orc.lib()   # noqa: F841  (loads and, if needed, builds the oracle)
    cores = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
    per = {}
    r = 3072  # sampled rows of each operand for the large workloads

    def timed(name, flops, sample, fn):
        t0 = time.time()
        fn()
        secs = time.time() - t0
        per[name] = {"tflops": round(flops / secs / 1e12, 8), "seconds": round(secs, 3), "gemm_flop": flops,
                     "sample": sample}

    def per_tensor():
        qa, sa = orc.quantize_tensor_current(h["a1"], 0)
        qb, sb = orc.quantize_tensor_current(h["b1"], 0, transpose=True)
        orc.gemm_ref(orc.dequantize(0, qa, 0, None, sa), orc.dequantize(0, qb, 0, None, sb))
    timed("per-tensor 16x32x64", 2 * 16 * 64 * 32, "whole workload", per_tensor)

    rd = 256
    def delayed():
        scale_a, scale_b = np.ones(1, np.float32), np.ones(1, np.float32)
        ha, hb = np.zeros(1024, np.float32), np.zeros(1024, np.float32)
        qa, _ = orc.delayed_step(h["A2"], 0, scale_a, ha)
        qb, _ = orc.delayed_step(h["B2"], 0, scale_b, hb, transpose=True)
        orc.gemm_ref(orc.dequantize(0, np.ascontiguousarray(qa[:rd]), 0, None, scale_a[0]),
                     orc.dequantize(0, qb, 0, None, scale_b[0]))
    timed("delayed 1024x2048x1024", 2 * rd * 1024 * 2048,
          "one step: both whole casts and history updates, GEMM of %d rows x all 1024 columns" % rd, delayed)

    def fine():
        qx, sx = orc.quantize_block(np.ascontiguousarray(h["X3"][:r]), 0, 1, 128)
        qw, sw = orc.quantize_block(np.ascontiguousarray(h["W3"][:128]), 0, 128, 128)
        orc.gemm_ref(orc.dequantize(1, qx, 0, sx, None, block=(1, 128)),
                     orc.dequantize(1, qw, 0, sw, None, block=(128, 128)))
    timed("fine-grained 4096x7168x2048", 2 * r * 128 * 7168,
          "%d rows of X, one 128-row weight block, their %d x 128 GEMM" % (r, r), fine)

    def mx():
        qa, ea = orc.quantize_mx(np.ascontiguousarray(h["A4"][:r]), 0)
        qb, eb = orc.quantize_mx(np.ascontiguousarray(h["B4"][:r]), 0)
        orc.gemm_ref(orc.dequantize(2, qa, 0, ea), orc.dequantize(2, qb, 0, eb))
    timed("MXFP8 8192^3", 2 * r * r * 8192, "%d rows of A and of B, their %d x %d GEMM" % (r, r, r), mx)

    def moss():
        S = {n: orc.compute_scale(orc.amax(h[k]), f, 1.0) for n, k, f in (("X", "X5", 0), ("W", "W5", 0), ("G", "G5", 1))}
        qX, eX = orc.quantize_moss_given(np.ascontiguousarray(h["X5"][:r]), 0, S["X"])
        qW, eW = orc.quantize_moss_given(np.ascontiguousarray(h["W5"][:r]), 0, S["W"])
        qG, eG = orc.quantize_moss_given(np.ascontiguousarray(h["G5"][:r]), 1, S["G"])
        qWT, eWT = orc.quantize_moss_given(np.ascontiguousarray(h["W5"][:, :r]), 0, S["W"], transpose=True)
        qGT, eGT = orc.quantize_moss_given(np.ascontiguousarray(h["G5"][:, :r]), 1, S["G"], transpose=True)
        qXT, eXT = orc.quantize_moss_given(np.ascontiguousarray(h["X5"][:, :r]), 0, S["X"], transpose=True)
        d = lambda q, e, f, s: orc.dequantize(3, q, f, e, s)
        orc.gemm_ref(d(qX, eX, 0, S["X"]), d(qW, eW, 0, S["W"]))
        orc.gemm_ref(d(qG, eG, 1, S["G"]), d(qWT, eWT, 0, S["W"]))
        orc.gemm_ref(d(qGT, eGT, 1, S["G"]), d(qXT, eXT, 0, S["X"]))
    timed("MOSS fwd+bwd 16384x4096x4096", 2 * r * r * 4096 * 2 + 2 * r * r * 16384,
          "global factors over whole tensors, %d-row samples of all six copies, the three GEMMs over them" % r, moss)

    flops = sum(v["gemm_flop"] for v in per.values())
    secs = sum(v["seconds"] for v in per.values())
    baseline = {"value": round(flops / secs / 1e12, 8), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
                "seconds": round(secs, 2), "per_config": per,
                "sample": ("oracle quantize + fp64 GEMM over a bounded sample of every workload (see per_config); "
                           "value = sampled GEMM flops over the summed oracle time")}

    # quantization SNR (dB, fp64 over whole tensors) of the operands the GPU step quantized
    def snr(bits, mode, q, e, fmt, S=None, block=(128, 128)):
        if mode == 1:
            xhat = orc.dequantize(mode, q.cpu().numpy(), fmt, e.cpu().numpy(), None, block=block)
        else:
            xhat = orc.dequantize(mode, q.cpu().numpy(), fmt, e.cpu().numpy(), S)
        return round(orc.snr_db(wl.bf16_bits_to_f32(bits), xhat), 3)

    S5 = {n: np.float32(o["S5" + n].item()) for n in ("X", "W", "G")}
    snr_db = {"fine-grained X 4096x7168 (1x128, 0.1% x50 outliers)": snr(h["X3"], 1, o["q3x"], o["s3x"], 0, block=(1, 128)),
              "fine-grained W 2048x7168 (128x128)": snr(h["W3"], 1, o["q3w"], o["s3w"], 0),
              "MXFP8 A 8192x8192 (MX)": snr(h["A4"], 2, o["q4a"], o["e4a"], 0),
              "MXFP8 B 8192x8192 (MX)": snr(h["B4"], 2, o["q4b"], o["e4b"], 0),
              "MOSS X 16384x4096 (MOSS, E4M3)": snr(h["X5"], 3, o["q5X"], o["e5X"], 0, S5["X"]),
              "MOSS W 4096x4096 (MOSS, E4M3)": snr(h["W5"], 3, o["q5W"], o["e5W"], 0, S5["W"]),
              "MOSS dY 16384x4096 (MOSS, E5M2)": snr(h["G5"], 3, o["q5G"], o["e5G"], 1, S5["G"])}
    return baseline, snr_db


if __name__ == "__main__":
    main()
