"""Benchmark of the decode hot path: fused QKV GEMV + fused gate+up+SwiGLU GEMV at M = 1
on 14B-shaped layers (hidden 5120, 40 q heads / 8 kv heads of 128, intermediate 13824),
u4 group-64 weights, seeded synthetic inputs resident in HBM.

One step = one fused-QKV call and one fused-gate+up call on the next layer of a
48-layer rotating pool (4.8 GB, far above the 256 MB last-level cache), each step
with its own activation vector.  The timed region replays a HIP graph holding all
K steps, bracketed by device synchronisation; the value is algorithmic bytes moved
per second (packed codes + bf16 scales/biases + activations + outputs).

Prints one JSON line (see the design doc for the fields).
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, published


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--pool", type=int, default=48, help="layer copies in the rotating weight pool")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-steps", type=int, default=6)
    ap.add_argument("--kernel-reps", type=int, default=1000,
                    help="launches per graph when timing one kernel on its own")
    return ap.parse_args()


KERNEL_SOURCES = ["gemm_affine_u4_amd/csrc/gemv_u4.hip", "gemm_affine_u4_amd/csrc/qmm_device.h"]
COUNTERS_SUMMARY = "profiles/gemv_u4_decode_14B_hbm_counters.md"


def counted_traffic(key: str):
    """HBM bytes per launch measured by the committed counter runs (FETCH_SIZE and
    WRITE_SIZE, calibrated on a device copy), or None if the kernel sources changed
    since they were taken."""
    import hashlib
    import re
    try:
        text = open(os.path.join(ROOT, COUNTERS_SUMMARY)).read()
        h = hashlib.sha256()
        for f in KERNEL_SOURCES:
            h.update(open(os.path.join(ROOT, f), "rb").read())
        if re.search(r"source_sha256_16: (\w+)", text).group(1) != h.hexdigest()[:16]:
            return None
        return int(re.search(rf"traffic_bytes_per_launch\.{key}: (\d+)", text).group(1))
    except (OSError, AttributeError):
        return None


def weight_bytes(rows: int, K: int) -> int:
    return rows * K // 2 + 2 * rows * (K // 64) * 2


def main():
    args = _args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1",
                          "n_gpus_requested": args.gpus}))
        sys.exit(2)

    import torch
    import gemm_affine_u4_amd as qmm
    import synth

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    qmm.load_library()
    dev = torch.device("cuda:0")
    sh = synth.DENSE_14B
    K, I, q_out, kv_out = sh.K, sh.I, sh.q_out, sh.kv_out
    rows_qkv, rows_gu = sh.qkv_rows, 2 * I

    # ---- inputs: one seeded layer, replicated into a rotating pool --------------------
    w_qkv = synth.gen_weight(synth.CFG_14B, 0, synth.PROJ_QKV, rows_qkv, K)
    w_gu = synth.gen_weight(synth.CFG_14B, 0, synth.PROJ_GATE_UP, rows_gu, K)

    def up(a):
        return torch.from_numpy(a.view(np.int32) if a.dtype == np.uint32 else a.view(np.int16)).to(dev)

    def pool_of(w, P):
        out = []
        for arr in (w.codes, w.scales, w.biases):
            t = up(arr)
            stack = torch.empty((P,) + tuple(t.shape), dtype=t.dtype, device=dev)
            stack.copy_(t.unsqueeze(0).expand_as(stack))
            out.append(stack)
        return out

    P = args.pool
    pq = pool_of(w_qkv, P)
    pg = pool_of(w_gu, P)
    NX = 16
    xs = torch.from_numpy(np.concatenate([synth.gen_x(synth.CFG_14B, 0, s, 1, K) for s in range(NX)]).view(np.int16)).to(dev)
    q = torch.empty((1, q_out), dtype=torch.bfloat16, device=dev)
    k = torch.empty((1, kv_out), dtype=torch.bfloat16, device=dev)
    v = torch.empty((1, kv_out), dtype=torch.bfloat16, device=dev)
    h = torch.empty((1, I), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    bytes_qkv = weight_bytes(rows_qkv, K) + K * 2 + rows_qkv * 2
    bytes_gu = weight_bytes(rows_gu, K) + K * 2 + I * 2
    bytes_step = bytes_qkv + bytes_gu

    stream = torch.cuda.Stream()

    def step(i):
        L = i % P
        x = xs[i % NX]
        qmm.qmm_fused_qkv(x, pq[0][L], pq[1][L], pq[2][L], q, k, v, stream=stream)
        qmm.qmm_fused_gate_up_swiglu(x, pg[0][L], pg[1][L], pg[2][L], h, stream=stream)

    def gate_up_only(i):
        L = i % P
        qmm.qmm_fused_gate_up_swiglu(xs[i % NX], pg[0][L], pg[1][L], pg[2][L], h, stream=stream)

    def qkv_only(i):
        L = i % P
        qmm.qmm_fused_qkv(xs[i % NX], pq[0][L], pq[1][L], pq[2][L], q, k, v, stream=stream)

    def capture(fn, n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            fn(0)  # touch once outside capture
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=stream):
                for i in range(n):
                    fn(i)
        torch.cuda.synchronize()
        return g

    def timed_replay(g, reps=1):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            e0.record(stream)
            for _ in range(reps):
                g.replay()
            e1.record(stream)
        e1.synchronize()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)  # ms

    # warmup (eager), then the timed graph of exactly K steps
    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            step(i)
    torch.cuda.synchronize()
    g_step = capture(step, args.steps)
    with torch.cuda.stream(stream):
        g_step.replay()
    torch.cuda.synchronize()
    ms_total = timed_replay(g_step)
    ms_per_step = ms_total / args.steps
    value = bytes_step / (ms_per_step * 1e-3) / 1e9

    # per-kernel average duration of the dominant kernel (gate+up GEMV), same stream
    n_k = args.kernel_reps
    g_gu = capture(gate_up_only, n_k)
    timed_replay(g_gu)
    ms_gu = timed_replay(g_gu) / n_k
    g_qkv = capture(qkv_only, n_k)
    timed_replay(g_qkv)
    ms_qkv = timed_replay(g_qkv) / n_k
    ach_gu = bytes_gu / (ms_gu * 1e-3) / 1e9
    ach_qkv = bytes_qkv / (ms_qkv * 1e-3) / 1e9

    # plain device copy of 2 GB: the read+write ceiling a simple kernel reaches
    src = torch.empty(1 << 30, dtype=torch.int16, device=dev)
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        dst.copy_(src)
    e1.record()
    e1.synchronize()
    copy_gbs = 10 * 2 * src.numel() * 2 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst

    result = {
        "metric": "achieved HBM GB/s (% of peak) fused u4 GEMV M=1; prefill GEMM TFLOP/s",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u4 weights, bf16 activations, fp32 accumulate",
        "data": "synthetic (seeded: codes uniform 0..15, scales U[0.001,0.01] bf16, bias=-8*scale, x~N(0,1) bf16)",
        "config": {"workload": "14B-shaped decode M=1: fused QKV [7168 x 5120] + fused gate+up+SwiGLU "
                               "[27648 x 5120], u4 g64, 48-layer rotating pool",
                   "global_batch": 1, "seq_len": 1, "parallelism": "none (1 GPU)",
                   "bytes_per_step": bytes_step, "pool_layers": P},
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "roofline": {"bound": "hbm", "kernel": "gemv_u4_kernel (fused gate+up+SwiGLU, K=5120)",
                     "achieved": round(ach_gu, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(ach_gu / HBM_PEAK_GBS, 4), "traffic": counted_traffic("gate_up"),
                     "bytes_per_launch": bytes_gu, "avg_launch_us": ms_gu * 1e3},
        "kernels": {"fused_qkv_gemv": {"avg_launch_us": ms_qkv * 1e3, "GB/s": round(ach_qkv, 1),
                                       "bytes_per_launch": bytes_qkv},
                    "fused_gate_up_gemv": {"avg_launch_us": ms_gu * 1e3, "GB/s": round(ach_gu, 1),
                                           "bytes_per_launch": bytes_gu}},
        "device_copy_GBps": round(copy_gbs, 1),
    }

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args.cpu_sample_steps, w_qkv, w_gu, bytes_step)

    print(json.dumps(result), flush=True)


def cpu_baseline(n_steps, w_qkv, w_gu, bytes_step):
    """The fp64 oracle, as it stands, on the same layer: n_steps full decode steps."""
    from threadpoolctl import threadpool_limits
    import synth
    from oracle import qmm_oracle as orc

    sh = synth.DENSE_14B
    x = synth.gen_x(synth.CFG_14B, 0, 0, 1, sh.K)
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        for _ in range(n_steps):
            orc.fused_qkv(x, w_qkv.codes, w_qkv.scales, w_qkv.biases, sh.q_out, sh.kv_out)
            orc.gate_up_swiglu(x, w_gu.codes, w_gu.scales, w_gu.biases, sh.I)
        dt = time.perf_counter() - t0
    return {"value": round(bytes_step * n_steps / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{n_steps} full 14B-shaped decode steps (fused QKV + gate+up+SwiGLU), fp64 NumPy, "
                      f"BLAS limited to 1 thread; {dt:.1f} s",
            "host": platform.processor() or platform.machine(), "host_cpus": os.cpu_count()}


if __name__ == "__main__":
    main()
